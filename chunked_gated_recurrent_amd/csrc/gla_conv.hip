// gla_conv.hip -- the short causal convolution in front of the mixer: every
// channel of the residual stream passes through a causal Conv1d of width 4
// followed by SiLU (Laplace 3B / Trainium2 page, section on normalisation
// and convolution), for prefill and for one decode step with a 4-row window
// of the most recent inputs.
//
//   z_t[c] = bias[c] + sum_{j<4} w[c][j] x_{t-3+j}[c],   y_t = z_t / (1 + e^-z_t)
//
// Both kernels are HBM streams: every input and output element moves once
// (prefill re-reads the 3 tokens before each run of tokens). A thread owns
// 16 bytes of channels (8 bf16 or 4 fp32) and keeps the 4-token window in
// registers in fp32.
#include "gla_device.h"

namespace gla {

constexpr int kConvK = 4;     // taps
constexpr int kConvRun = 32;  // tokens per prefill thread
// decode grid: three 256-thread workgroups per CU of the 256 (the bf16
// kernel's 130 VGPRs leave room for three waves per SIMD); measured against
// 2 and 4 per CU and against one sequence per thread: 29.8 us per step at
// 1,280 x 3,072 against 35.2, 31.9 and 36.0 us
constexpr long long kConvDecodeThreads = 3 * 256 * 256;

template <typename Tin>
struct ConvVec {
  static constexpr int N = 16 / sizeof(Tin);  // channels per thread
};

template <typename Tin>
__device__ __forceinline__ void load_vec(const Tin *p, float (&out)[ConvVec<Tin>::N]) {
  constexpr int N = ConvVec<Tin>::N;
  typedef Tin vec_t __attribute__((ext_vector_type(N)));
  const vec_t v = *reinterpret_cast<const vec_t *>(p);
#pragma unroll
  for (int e = 0; e < N; ++e) out[e] = (float)v[e];
}

template <typename Tin>
__device__ __forceinline__ void store_vec(Tin *p, const float (&in)[ConvVec<Tin>::N]) {
  constexpr int N = ConvVec<Tin>::N;
  typedef Tin vec_t __attribute__((ext_vector_type(N)));
  vec_t v;
#pragma unroll
  for (int e = 0; e < N; ++e) v[e] = (Tin)in[e];
  *reinterpret_cast<vec_t *>(p) = v;
}

// SiLU with the hardware exponential and reciprocal (about 1 ulp each); a
// full-precision division would make the prefill ALU-bound. For z -> -inf
// the reciprocal of inf is 0, so the result tends to (-)0 as it should.
__device__ __forceinline__ float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// One thread: channels [c, c + N) of batch entry b over tokens
// [r * kConvRun, min(T, (r + 1) * kConvRun)).
template <typename Tin>
__global__ __launch_bounds__(256) void short_conv_fwd_kernel(
    const Tin *__restrict__ x, const float *__restrict__ w,
    const float *__restrict__ bias, const float *__restrict__ win_in,
    Tin *__restrict__ y, float *__restrict__ win_out, int B, int T, int D) {
  constexpr int N = ConvVec<Tin>::N;
  const int groups = D / N;
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  const int runs = (T + kConvRun - 1) / kConvRun;
  if (gid >= (long long)B * runs * groups) return;
  const int cg = (int)(gid % groups);
  const long long br = gid / groups;
  const int r = (int)(br % runs);
  const int b = (int)(br / runs);
  const int c = cg * N;
  const int t0 = r * kConvRun, t1 = min(T, t0 + kConvRun);

  typedef float f32x4n __attribute__((ext_vector_type(4)));
  float wt[kConvK][N], bs[N];
#pragma unroll
  for (int e = 0; e < N; ++e) {
    const f32x4n wv = *reinterpret_cast<const f32x4n *>(w + (long long)(c + e) * kConvK);
#pragma unroll
    for (int j = 0; j < kConvK; ++j) wt[j][e] = wv[j];
    bs[e] = bias ? bias[c + e] : 0.f;
  }
  // window: the kConvK inputs before t0, oldest first
  float win[kConvK][N];
#pragma unroll
  for (int j = 0; j < kConvK; ++j) {
    const int t = t0 - kConvK + j;
    if (t >= 0) {
      load_vec(x + ((long long)b * T + t) * D + c, win[j]);
    } else if (win_in) {
      const float *src = win_in + ((long long)b * kConvK + (kConvK + t)) * D + c;
#pragma unroll
      for (int e = 0; e < N; ++e) win[j][e] = src[e];
    } else {
#pragma unroll
      for (int e = 0; e < N; ++e) win[j][e] = 0.f;
    }
  }
  auto step = [&](const float (&xt)[N], int t) {
    float out[N];
#pragma unroll
    for (int e = 0; e < N; ++e) {
      win[0][e] = win[1][e];
      win[1][e] = win[2][e];
      win[2][e] = win[3][e];
      win[3][e] = xt[e];
      float z = bs[e];
#pragma unroll
      for (int j = 0; j < kConvK; ++j) z = fmaf(wt[j][e], win[j][e], z);
      out[e] = silu(z);
    }
    store_vec(y + ((long long)b * T + t) * D + c, out);
  };
  if (t1 - t0 == kConvRun) {
    // a full run: blocks of 8 tokens whose loads go out together, the next
    // block's before the current one is computed (straight-line code)
    constexpr int BLK = 8;
    float xa[BLK][N], xb[BLK][N];
    // (the scheduling barriers keep the compiler from sinking each block's
    // loads down to their uses, which would leave one load in flight)
#pragma unroll
    for (int i = 0; i < BLK; ++i) load_vec(x + ((long long)b * T + t0 + i) * D + c, xa[i]);
#pragma unroll
    for (int blk = 0; blk < kConvRun; blk += 2 * BLK) {
#pragma unroll
      for (int i = 0; i < BLK; ++i)
        load_vec(x + ((long long)b * T + t0 + blk + BLK + i) * D + c, xb[i]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < BLK; ++i) step(xa[i], t0 + blk + i);
      if (blk + 2 * BLK < kConvRun) {
#pragma unroll
        for (int i = 0; i < BLK; ++i)
          load_vec(x + ((long long)b * T + t0 + blk + 2 * BLK + i) * D + c, xa[i]);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < BLK; ++i) step(xb[i], t0 + blk + BLK + i);
    }
  } else {
    for (int t = t0; t < t1; ++t) {
      float xt[N];
      load_vec(x + ((long long)b * T + t) * D + c, xt);
      step(xt, t);
    }
  }
  if (win_out && t1 == T) {  // the run holding the sequence's last token
#pragma unroll
    for (int j = 0; j < kConvK; ++j) {
      float *dst = win_out + ((long long)b * kConvK + j) * D + c;
#pragma unroll
      for (int e = 0; e < N; ++e) dst[e] = win[j][e];
    }
  }
}

// One decode step: the window [N, kConvK, D] shifts by one token in place.
// A thread keeps one channel group (and its taps) and walks sequences n0,
// n0 + stride, ...; the next sequence's window rows and token are loaded
// before the current one is computed and stored, so each thread always has
// a read in flight beside its writes (one pass per thread would run the
// whole grid through a read phase and then a write phase).
template <typename Tin>
__global__ __launch_bounds__(256) void short_conv_decode_kernel(
    const Tin *__restrict__ x, const float *__restrict__ w,
    const float *__restrict__ bias, float *__restrict__ window,
    Tin *__restrict__ y, int Nseq, int D, int stride) {
  constexpr int N = ConvVec<Tin>::N;
  typedef float f32x4n __attribute__((ext_vector_type(4)));
  const int groups = D / N;
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  const int cg = (int)(gid % groups);
  const long long n0 = gid / groups;
  if (n0 >= stride || n0 >= Nseq) return;
  const int c = cg * N;
  // the taps of channel c + e are the 16 bytes at w + 4 (c + e)
  f32x4n wt[N];
  float bs[N];
#pragma unroll
  for (int e = 0; e < N; ++e) {
    wt[e] = *reinterpret_cast<const f32x4n *>(w + (long long)(c + e) * kConvK);
    bs[e] = bias ? bias[c + e] : 0.f;
  }
  struct Stage {
    float win[kConvK - 1][N], xt[N];
  };
  auto load = [&](long long n, Stage &st) {
    load_vec(x + n * D + c, st.xt);
#pragma unroll
    for (int j = 1; j < kConvK; ++j) {
      const float *src = window + (n * kConvK + j) * D + c;
#pragma unroll
      for (int e = 0; e < N; e += 4) {
        const f32x4n v = __builtin_nontemporal_load(reinterpret_cast<const f32x4n *>(src + e));
        st.win[j - 1][e] = v[0];
        st.win[j - 1][e + 1] = v[1];
        st.win[j - 1][e + 2] = v[2];
        st.win[j - 1][e + 3] = v[3];
      }
    }
  };
  auto finish = [&](long long n, const Stage &st) {
    float out[N];
#pragma unroll
    for (int e = 0; e < N; ++e) {
      float z = bs[e];
#pragma unroll
      for (int j = 0; j < kConvK - 1; ++j) z = fmaf(wt[e][j], st.win[j][e], z);
      z = fmaf(wt[e][kConvK - 1], st.xt[e], z);
      out[e] = silu(z);
    }
#pragma unroll
    for (int j = 0; j < kConvK; ++j) {
      float *dst = window + (n * kConvK + j) * D + c;
#pragma unroll
      for (int e = 0; e < N; e += 4) {
        f32x4n v;
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = j < kConvK - 1 ? st.win[j][e + u] : st.xt[e + u];
        __builtin_nontemporal_store(v, reinterpret_cast<f32x4n *>(dst + e));
      }
    }
    store_vec(y + n * D + c, out);
  };
  Stage a, b;
  load(n0, a);
  long long n = n0;
  while (true) {  // two stages, swapped by unrolling
    const long long n1 = n + stride;
    if (n1 < Nseq) load(n1, b);
    finish(n, a);
    if (n1 >= Nseq) break;
    const long long n2 = n1 + stride;
    if (n2 < Nseq) load(n2, a);
    finish(n1, b);
    if (n2 >= Nseq) break;
    n = n2;
  }
}

hipError_t launch_short_conv_fwd(int dt, int B, int T, int D, const void *x,
                                 const float *w, const float *bias, const float *win_in,
                                 void *y, float *win_out, hipStream_t s) {
  const int runs = (T + kConvRun - 1) / kConvRun;
  if (dt == 1) {
    const long long n = (long long)B * runs * (D / ConvVec<bf16>::N);
    hipLaunchKernelGGL(short_conv_fwd_kernel<bf16>, dim3((unsigned)((n + 255) / 256)),
                       dim3(256), 0, s, (const bf16 *)x, w, bias, win_in, (bf16 *)y,
                       win_out, B, T, D);
  } else {
    const long long n = (long long)B * runs * (D / ConvVec<float>::N);
    hipLaunchKernelGGL(short_conv_fwd_kernel<float>, dim3((unsigned)((n + 255) / 256)),
                       dim3(256), 0, s, (const float *)x, w, bias, win_in, (float *)y,
                       win_out, B, T, D);
  }
  return hipGetLastError();
}

hipError_t launch_short_conv_decode(int dt, int N, int D, const void *x, const float *w,
                                    const float *bias, float *window, void *y,
                                    hipStream_t s) {
  // each thread walks every stride-th sequence of one channel group
  // (N >= 1 here)
  const int groups = D / (dt == 1 ? ConvVec<bf16>::N : ConvVec<float>::N);
  const long long per = (kConvDecodeThreads + groups - 1) / groups;
  const int stride = (int)(per < N ? per : N);
  const long long n = (long long)stride * groups;
  if (dt == 1)
    hipLaunchKernelGGL(short_conv_decode_kernel<bf16>, dim3((unsigned)((n + 255) / 256)),
                       dim3(256), 0, s, (const bf16 *)x, w, bias, window, (bf16 *)y, N, D,
                       stride);
  else
    hipLaunchKernelGGL(short_conv_decode_kernel<float>, dim3((unsigned)((n + 255) / 256)),
                       dim3(256), 0, s, (const float *)x, w, bias, window, (float *)y, N, D,
                       stride);
  return hipGetLastError();
}

}  // namespace gla
