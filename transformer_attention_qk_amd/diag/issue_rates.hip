// Issue-rate probe of one gfx950 compute unit (a diagnostic, not part of the attention library):
// loops of independent instructions, written in inline assembly so the compiler keeps their
// order, timed per wave with the shader clock (s_memtime). It answers the questions the forward
// kernel's design turns on: does a wave's vector work run while its own MFMAs run, and which
// vector instructions hold the matrix pipe. Only ALU instructions run inside the timed loops;
// their values are discarded (they may be inf or NaN), and hazards between them do not matter
// because nothing reads their results except the next iteration of the same instructions.
//
// extern "C" int attn_diag_issue_rates(double* cycles, int n):
//   cycles: HOST array of n >= 2 * kModes doubles; cycles[2 m + w] is the cycles per loop
//   iteration (the maximum over the waves) of mode m with w + 1 waves per SIMD (a workgroup of
//   256 or 512 threads on one compute unit). Returns 0, or a HIP error code.
// extern "C" const char* attn_diag_issue_name(int m): the mode's description, or NULL.
#include <hip/hip_runtime.h>

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kModes = 9;
const char* const kNames[kModes] = {
    "16 mfma 32x32x16 bf16 (4 chains)",
    "16 mfma (1 chain)",
    "32 v_exp_f32",
    "64 v_fma_f32",
    "16 mfma + 32 v_exp_f32 interleaved",
    "16 mfma + 64 v_fma_f32 interleaved",
    "16 mfma + 16 v_cvt_pk_bf16_f32 interleaved",
    "16 mfma + 16 v_dot2c_f32_bf16 interleaved",
    "16 mfma + 64 add/shift/and interleaved",
};

#define MF(acc) "v_mfma_f32_32x32x16_bf16 " acc ", %[a], %[b], " acc "\n"
#define EX(r) "v_exp_f32 " r ", " r "\n"
#define FM(r) "v_fma_f32 " r ", " r ", %[f], %[f]\n"
#define CV(r, x) "v_cvt_pk_bf16_f32 " x ", " r ", " r "\n"
#define DT(r, x) "v_dot2c_f32_bf16 " r ", " x ", " x "\n"
#define AD(r, x) "v_add_f32 " r ", " r ", " x "\n" "v_lshlrev_b32 " x ", 16, " x "\n" \
                 "v_add_f32 " r ", " r ", " x "\n" "v_and_b32 " x ", 0xffff0000, " x "\n"
#define C4 "%[c0]", "%[c1]", "%[c2]", "%[c3]"
#define ACC : [c0] "+v"(c0), [c1] "+v"(c1), [c2] "+v"(c2), [c3] "+v"(c3)
#define E16 , [e0] "+v"(e[0]), [e1] "+v"(e[1]), [e2] "+v"(e[2]), [e3] "+v"(e[3]), \
    [e4] "+v"(e[4]), [e5] "+v"(e[5]), [e6] "+v"(e[6]), [e7] "+v"(e[7]), [e8] "+v"(e[8]), \
    [e9] "+v"(e[9]), [e10] "+v"(e[10]), [e11] "+v"(e[11]), [e12] "+v"(e[12]), \
    [e13] "+v"(e[13]), [e14] "+v"(e[14]), [e15] "+v"(e[15])
#define IN : [a] "v"(a), [b] "v"(b), [f] "v"(seed)
// the 16 products of one iteration, 4 chains
#define M16 MF("%[c0]") MF("%[c1]") MF("%[c2]") MF("%[c3]") MF("%[c0]") MF("%[c1]") MF("%[c2]") \
    MF("%[c3]") MF("%[c0]") MF("%[c1]") MF("%[c2]") MF("%[c3]") MF("%[c0]") MF("%[c1]")       \
    MF("%[c2]") MF("%[c3]")
// one product followed by vector work X(i), for the 16 products
#define G16(X) MF("%[c0]") X(0) MF("%[c1]") X(1) MF("%[c2]") X(2) MF("%[c3]") X(3)           \
    MF("%[c0]") X(4) MF("%[c1]") X(5) MF("%[c2]") X(6) MF("%[c3]") X(7) MF("%[c0]") X(8)     \
    MF("%[c1]") X(9) MF("%[c2]") X(10) MF("%[c3]") X(11) MF("%[c0]") X(12) MF("%[c1]") X(13) \
    MF("%[c2]") X(14) MF("%[c3]") X(15)
#define R(i) "%[e" #i "]"
#define X_EXP(i) EX(R(i)) EX(R(i))
#define X_FMA(i) FM(R(i)) FM(R(i)) FM(R(i)) FM(R(i))
#define X_CVT(i) CV(R(i), "%[x]")
#define X_DOT(i) DT(R(i), "%[x]")
#define X_ADD(i) AD(R(i), "%[x]")
#define V16(X) X(0) X(1) X(2) X(3) X(4) X(5) X(6) X(7) X(8) X(9) X(10) X(11) X(12) X(13) X(14) X(15)

template <int MODE>
__global__ void probe(long long* out, float seed, int iters) {
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(seed * i);
    b[i] = (__bf16)(seed + i);
  }
  float e[16];
  for (int i = 0; i < 16; ++i) e[i] = seed * (float)(threadIdx.x + i);
  float x = seed;
  const long long t0 = __builtin_readcyclecounter();
  for (int it = 0; it < iters; ++it) {
    if constexpr (MODE == 0) {
      asm volatile(M16 ACC IN);
    } else if constexpr (MODE == 1) {
      asm volatile(MF("%[c0]") MF("%[c0]") MF("%[c0]") MF("%[c0]") MF("%[c0]") MF("%[c0]")
                   MF("%[c0]") MF("%[c0]") MF("%[c0]") MF("%[c0]") MF("%[c0]") MF("%[c0]")
                   MF("%[c0]") MF("%[c0]") MF("%[c0]") MF("%[c0]") ACC IN);
    } else if constexpr (MODE == 2) {
      asm volatile(V16(X_EXP) ACC E16 IN);
    } else if constexpr (MODE == 3) {
      asm volatile(V16(X_FMA) ACC E16 IN);
    } else if constexpr (MODE == 4) {
      asm volatile(G16(X_EXP) ACC E16 IN);
    } else if constexpr (MODE == 5) {
      asm volatile(G16(X_FMA) ACC E16 IN);
    } else if constexpr (MODE == 6) {
      asm volatile(G16(X_CVT) ACC E16, [x] "+v"(x) IN);
    } else if constexpr (MODE == 7) {
      asm volatile(G16(X_DOT) ACC E16, [x] "+v"(x) IN);
    } else {
      asm volatile(G16(X_ADD) ACC E16, [x] "+v"(x) IN);
    }
  }
  const long long t1 = __builtin_readcyclecounter();
  float s = x;
  for (int i = 0; i < 16; ++i) s += e[i] + c0[i] + c1[i] + c2[i] + c3[i];
  // one slot per wave of the one workgroup (at most 8 waves); the sum keeps the values live
  if ((threadIdx.x & 63) == 0) out[threadIdx.x / 64] = (t1 - t0) + (s == 1.2345f ? 1 : 0);
}

template <int MODE>
hipError_t run(long long* d_out, int threads, int iters) {
  hipLaunchKernelGGL(probe<MODE>, dim3(1), dim3(threads), 0, 0, d_out, 0.001f, iters);
  return hipGetLastError();
}

hipError_t run_mode(int m, long long* d_out, int threads, int iters) {
  switch (m) {
    case 0: return run<0>(d_out, threads, iters);
    case 1: return run<1>(d_out, threads, iters);
    case 2: return run<2>(d_out, threads, iters);
    case 3: return run<3>(d_out, threads, iters);
    case 4: return run<4>(d_out, threads, iters);
    case 5: return run<5>(d_out, threads, iters);
    case 6: return run<6>(d_out, threads, iters);
    case 7: return run<7>(d_out, threads, iters);
    default: return run<8>(d_out, threads, iters);
  }
}

}  // namespace

extern "C" const char* attn_diag_issue_name(int m) {
  return (m >= 0 && m < kModes) ? kNames[m] : nullptr;
}

extern "C" int attn_diag_issue_rates(double* cycles, int n) {
  if (cycles == nullptr || n < 2 * kModes) return (int)hipErrorInvalidValue;
  long long* d = nullptr;
  hipError_t e = hipMalloc(&d, 8 * sizeof(long long));
  if (e != hipSuccess) return (int)e;
  const int iters = 2000;
  for (int m = 0; m < kModes && e == hipSuccess; ++m) {
    for (int w = 0; w < 2 && e == hipSuccess; ++w) {
      const int threads = 256 * (w + 1);  // one or two waves on each of the CU's 4 SIMDs
      double best = 0.0;
      for (int rep = 0; rep < 2 && e == hipSuccess; ++rep) {  // the first run warms up
        e = run_mode(m, d, threads, iters);
        if (e == hipSuccess) e = hipDeviceSynchronize();
        long long h[8] = {};
        if (e == hipSuccess) e = hipMemcpy(h, d, sizeof(h), hipMemcpyDeviceToHost);
        double mx = 0.0;
        for (int i = 0; i < threads / 64; ++i) mx = (double)h[i] > mx ? (double)h[i] : mx;
        best = mx / iters;
      }
      cycles[2 * m + w] = best;
    }
  }
  hipFree(d);
  return (int)e;
}
