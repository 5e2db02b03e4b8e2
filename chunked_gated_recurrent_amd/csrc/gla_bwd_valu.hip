// gla_bwd_valu.hip -- backward of the chunked Simple GLA forward on the
// vector ALUs, in fp32 arithmetic: fp32 inputs, and head sizes off the
// matrix-core path (any dk, dv the library accepts).
//
// Same gradients and chunk formulas as the matrix-core backward (Laplace 3B /
// Trainium2 page, sections "GLA mixer" and "Challenge 3"), with
// G_t = dL/dS_t = lambda G_{t+1} + scale q_t^T dO_t:
//     dq_i = scale (lambda^(i+1) dO_i S_prev^T + sum_{j<=i} lambda^(i-j) (dO_i . v_j) k_j)
//     dv_i = lambda^(L-1-i) k_i Ch + scale sum_{t>=i} lambda^(t-i) (q_t . k_i) dO_t
//     dk_i = lambda^(L-1-i) Ch v_i^T + scale sum_{t>=i} lambda^(t-i) (dO_t . v_i) q_t
//     Ch  <- lambda^L Ch + scale sum_t lambda^(t+1) q_t^T dO_t
// for chunks of L <= 32 tokens. A workgroup owns one (work item, head, dv
// tile of TV <= 64 columns) and keeps everything in LDS as fp32; dq and dk
// contract over dv, so each dv tile writes fp32 partial rows
// [dv tile][H][token][dk] that a streaming kernel sums into dq and dk.
#include "gla_device.h"

namespace gla {

constexpr int kBwdValuC = 32;  // tokens per chunk

namespace {

template <typename Tin>
__device__ __forceinline__ float ldf(const Tin *p) {
  return (float)(*p);
}

__device__ __forceinline__ float *vpart_row(float *part, int dtile, int h, long long t,
                                            int H, long long total_T, int dk) {
  return part + (((long long)dtile * H + h) * total_T + t) * dk;
}

}  // namespace

// dq pass: walks the item's chunks forward carrying the state tile S[:, tile].
template <typename Tin>
__global__ __launch_bounds__(256) void bwd_dq_valu_kernel(
    const Tin *__restrict__ k, const Tin *__restrict__ v, const Tin *__restrict__ dout,
    const float *__restrict__ s0, const float *__restrict__ slots,
    float *__restrict__ part_dq, Plan plan, Decay dec, float scale, int H, int dk,
    int dv, int TV) {
  constexpr int C = kBwdValuC;
  extern __shared__ float bsm[];
  float *sK = bsm;            // [C][dk]
  float *sV = sK + C * dk;    // [C][TV]
  float *sD = sV + C * TV;    // [C][TV]
  float *sP = sD + C * TV;    // [C][C]
  float *sS = sP + C * C;     // [dk][TV]
  float *sPow = sS + dk * TV; // [C+1] (+3)

  const int ndt = dv / TV;
  int unit, dtile;
  xcd_unit(plan, ndt, plan.max_items * H, unit, dtile);
  if (unit >= plan.max_items * H) return;
  const int slot = unit / H;
  const int h = unit - slot * H;
  int idx;
  Item it;
  if (!slot_item(plan, slot, idx, it)) return;
  const int tid = threadIdx.x;
  const int c0 = dtile * TV;
  const long long rowK = (long long)H * dk, rowV = (long long)H * dv;
  const int nch = (it.t1 - it.t0 + C - 1) / C;

  for (int n = tid; n <= C; n += blockDim.x) sPow[n] = pow_f64(dec.lam[h], n);
  {
    const float *src = (it.flags & kFirstSeg)
                           ? (s0 ? s0 + ((long long)it.n * H + h) * dk * dv : nullptr)
                           : slots + ((long long)(idx - 1) * H + h) * dk * dv;
    for (int e = tid; e < dk * TV; e += blockDim.x) {
      const int d = e / TV, c = e - d * TV;
      sS[e] = src ? src[(long long)d * dv + c0 + c] : 0.f;
    }
  }
  __syncthreads();

  for (int ch = 0; ch < nch; ++ch) {
    const int tb = it.t0 + ch * C;
    const int L = min(C, it.t1 - tb);
    for (int e = tid; e < C * dk; e += blockDim.x) {
      const int r = e / dk, d = e - r * dk;
      sK[e] = r < L ? ldf(k + (long long)(tb + r) * rowK + (long long)h * dk + d) : 0.f;
    }
    for (int e = tid; e < C * TV; e += blockDim.x) {
      const int r = e / TV, c = e - r * TV;
      const long long off = (long long)(tb + r) * rowV + (long long)h * dv + c0 + c;
      sV[e] = r < L ? ldf(v + off) : 0.f;
      sD[e] = r < L ? ldf(dout + off) : 0.f;
    }
    __syncthreads();
    // P'[i][j] = (dO_i . v_j over the tile) lambda^(i-j), j <= i
    for (int e = tid; e < C * C; e += blockDim.x) {
      const int i = e / C, j = e - i * C;
      float acc = 0.f;
      if (j <= i) {
        for (int c = 0; c < TV; ++c) acc = fmaf(sD[i * TV + c], sV[j * TV + c], acc);
        acc *= sPow[i - j];
      }
      sP[e] = acc;
    }
    __syncthreads();
    for (int e = tid; e < C * dk; e += blockDim.x) {
      const int i = e / dk, d = e - i * dk;
      if (i < L) {
        float inter = 0.f;
        for (int c = 0; c < TV; ++c) inter = fmaf(sD[i * TV + c], sS[d * TV + c], inter);
        float intra = 0.f;
        for (int j = 0; j <= i; ++j) intra = fmaf(sP[i * C + j], sK[j * dk + d], intra);
        vpart_row(part_dq, dtile, h, tb + i, H, plan.total_T, dk)[d] =
            scale * fmaf(sPow[i + 1], inter, intra);
      }
    }
    __syncthreads();
    const float lamL = sPow[L];
    for (int e = tid; e < dk * TV; e += blockDim.x) {
      const int d = e / TV, c = e - d * TV;
      float acc = 0.f;
      for (int j = 0; j < L; ++j) acc = fmaf(sPow[L - 1 - j] * sK[j * dk + d], sV[j * TV + c], acc);
      sS[e] = fmaf(lamL, sS[e], acc);
    }
    __syncthreads();
  }
}

// Reverse pass: walks the item's chunks backward carrying Ch[:, tile].
//   CARRY_ONLY: the local carry U of a time segment (Ch from zero, only the
//   Ch update), written to its slot; every item but a sequence's first.
template <typename Tin, bool CARRY_ONLY>
__global__ __launch_bounds__(256) void bwd_dkdv_valu_kernel(
    const Tin *__restrict__ q, const Tin *__restrict__ k, const Tin *__restrict__ v,
    const Tin *__restrict__ dout, const float *__restrict__ ds_final,
    float *__restrict__ cslots, Tin *__restrict__ dv_out, float *__restrict__ ds0,
    float *__restrict__ part_dk, Plan plan, Decay dec, float scale, int H, int dk,
    int dv, int TV) {
  constexpr int C = kBwdValuC;
  extern __shared__ float bsm[];
  float *sQ = bsm;             // [C][dk]
  float *sK = sQ + C * dk;     // [C][dk]
  float *sV = sK + C * dk;     // [C][TV]
  float *sD = sV + C * TV;     // [C][TV]
  float *sA = sD + C * TV;     // [C][C]  scale lambda^(t-i) q_t . k_i
  float *sB = sA + C * C;      // [C][C]  scale lambda^(t-i) dO_t . v_i
  float *sCh = sB + C * C;     // [dk][TV]
  float *sPow = sCh + dk * TV; // [C+1] (+3)

  const int ndt = dv / TV;
  int unit, dtile;
  xcd_unit(plan, ndt, plan.max_items * H, unit, dtile);
  if (unit >= plan.max_items * H) return;
  const int slot = unit / H;
  const int h = unit - slot * H;
  int idx;
  Item it;
  if (!slot_item(plan, slot, idx, it)) return;
  if (CARRY_ONLY && (it.flags & kFirstSeg)) return;  // no earlier item reads it
  const int tid = threadIdx.x;
  const int c0 = dtile * TV;
  const long long rowK = (long long)H * dk, rowV = (long long)H * dv;
  const int nch = (it.t1 - it.t0 + C - 1) / C;
  const long long state_off = ((long long)it.n * H + h) * dk * dv;

  for (int n = tid; n <= C; n += blockDim.x) sPow[n] = pow_f64(dec.lam[h], n);
  {
    const float *src = nullptr;
    if (!CARRY_ONLY)
      src = (it.flags & kLastSeg) ? (ds_final ? ds_final + state_off : nullptr)
                                  : cslots + ((long long)(idx + 1) * H + h) * dk * dv;
    for (int e = tid; e < dk * TV; e += blockDim.x) {
      const int d = e / TV, c = e - d * TV;
      sCh[e] = src ? src[(long long)d * dv + c0 + c] : 0.f;
    }
  }
  __syncthreads();

  for (int ch = nch - 1; ch >= 0; --ch) {
    const int tb = it.t0 + ch * C;
    const int L = min(C, it.t1 - tb);
    for (int e = tid; e < C * dk; e += blockDim.x) {
      const int r = e / dk, d = e - r * dk;
      const long long off = (long long)(tb + r) * rowK + (long long)h * dk + d;
      sQ[e] = r < L ? ldf(q + off) : 0.f;
      if (!CARRY_ONLY) sK[e] = r < L ? ldf(k + off) : 0.f;
    }
    for (int e = tid; e < C * TV; e += blockDim.x) {
      const int r = e / TV, c = e - r * TV;
      const long long off = (long long)(tb + r) * rowV + (long long)h * dv + c0 + c;
      sD[e] = r < L ? ldf(dout + off) : 0.f;
      if (!CARRY_ONLY) sV[e] = r < L ? ldf(v + off) : 0.f;
    }
    __syncthreads();
    if (!CARRY_ONLY) {
      for (int e = tid; e < C * C; e += blockDim.x) {
        const int t = e / C, i = e - t * C;
        float a = 0.f, b = 0.f;
        if (t >= i) {
          for (int d = 0; d < dk; ++d) a = fmaf(sQ[t * dk + d], sK[i * dk + d], a);
          for (int c = 0; c < TV; ++c) b = fmaf(sD[t * TV + c], sV[i * TV + c], b);
          const float wgt = scale * sPow[t - i];
          a *= wgt;
          b *= wgt;
        }
        sA[e] = a;
        sB[e] = b;
      }
      __syncthreads();
      for (int e = tid; e < C * TV; e += blockDim.x) {
        const int i = e / TV, c = e - i * TV;
        if (i < L) {
          float x = 0.f;
          for (int d = 0; d < dk; ++d) x = fmaf(sK[i * dk + d], sCh[d * TV + c], x);
          float y = 0.f;
          for (int t = i; t < L; ++t) y = fmaf(sA[t * C + i], sD[t * TV + c], y);
          dv_out[(long long)(tb + i) * rowV + (long long)h * dv + c0 + c] =
              (Tin)fmaf(sPow[L - 1 - i], x, y);
        }
      }
      for (int e = tid; e < C * dk; e += blockDim.x) {
        const int i = e / dk, d = e - i * dk;
        if (i < L) {
          float x = 0.f;
          for (int c = 0; c < TV; ++c) x = fmaf(sCh[d * TV + c], sV[i * TV + c], x);
          float y = 0.f;
          for (int t = i; t < L; ++t) y = fmaf(sB[t * C + i], sQ[t * dk + d], y);
          vpart_row(part_dk, dtile, h, tb + i, H, plan.total_T, dk)[d] =
              fmaf(sPow[L - 1 - i], x, y);
        }
      }
      __syncthreads();
    }
    const float lamL = sPow[L];
    for (int e = tid; e < dk * TV; e += blockDim.x) {
      const int d = e / TV, c = e - d * TV;
      float acc = 0.f;
      for (int t = 0; t < L; ++t) acc = fmaf(sPow[t + 1] * sQ[t * dk + d], sD[t * TV + c], acc);
      sCh[e] = fmaf(lamL, sCh[e], scale * acc);
    }
    __syncthreads();
  }

  float *dst = nullptr;
  if (CARRY_ONLY)
    dst = cslots + ((long long)idx * H + h) * dk * dv;
  else if ((it.flags & kFirstSeg) && ds0)
    dst = ds0 + state_off;  // after the first chunk Ch is dL/dS0
  if (dst)
    for (int e = tid; e < dk * TV; e += blockDim.x) {
      const int d = e / TV, c = e - d * TV;
      dst[(long long)d * dv + c0 + c] = sCh[e];
    }
}

// dq, dk <- sum of the dv-tile partials, in the input dtype, [tokens, H, dk].
// One thread per 4 consecutive values of one (token, head) row.
template <typename Tout>
__global__ __launch_bounds__(256) void bwd_reduce_valu_kernel(
    const float *__restrict__ part_dq, const float *__restrict__ part_dk,
    Tout *__restrict__ dq, Tout *__restrict__ dk, long long total_T, int H, int dkd,
    int ndt) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;  // float4 index
  const int per_row = dkd / 4;
  const long long n4 = total_T * H * per_row;
  if (e >= n4) return;
  const long long row = e / per_row;  // token * H + head
  const int c4 = (int)(e - row * per_row);
  const long long t = row / H;
  const int h = (int)(row - t * H);
  float4 sq = make_float4(0.f, 0.f, 0.f, 0.f), sk = sq;
  for (int d = 0; d < ndt; ++d) {
    const long long off = (((long long)d * H + h) * total_T + t) * dkd + 4 * c4;
    const float4 a = *reinterpret_cast<const float4 *>(part_dq + off);
    const float4 b = *reinterpret_cast<const float4 *>(part_dk + off);
    sq.x += a.x; sq.y += a.y; sq.z += a.z; sq.w += a.w;
    sk.x += b.x; sk.y += b.y; sk.z += b.z; sk.w += b.w;
  }
  Tout *oq = dq + row * dkd + 4 * c4, *ok = dk + row * dkd + 4 * c4;
  oq[0] = (Tout)sq.x; oq[1] = (Tout)sq.y; oq[2] = (Tout)sq.z; oq[3] = (Tout)sq.w;
  ok[0] = (Tout)sk.x; ok[1] = (Tout)sk.y; ok[2] = (Tout)sk.z; ok[3] = (Tout)sk.w;
}

int valu_bwd_tile(int dv) {
  const int m = dv / 16;
  for (int t = 4; t > 1; --t)
    if (m % t == 0) return 16 * t;
  return 16;
}

size_t valu_bwd_lds_dq(int dk, int TV) {
  constexpr int C = kBwdValuC;
  return sizeof(float) * ((size_t)C * dk + 2 * C * TV + C * C + (size_t)dk * TV + C + 4);
}

size_t valu_bwd_lds_dkdv(int dk, int TV) {
  constexpr int C = kBwdValuC;
  return sizeof(float) * ((size_t)2 * C * dk + 2 * C * TV + 2 * C * C + (size_t)dk * TV + C + 4);
}

template <typename Tin>
static void launch_bwd_valu_t(const Plan &p, const BwdArgs &a, const Decay &dec,
                              hipStream_t s) {
  const int TV = valu_bwd_tile(a.dv), dkd = a.dk_dim;
  const unsigned grid = xcd_grid(p.deal, (long long)p.max_items * a.H, a.dv / TV);
  const size_t lq = valu_bwd_lds_dq(dkd, TV), lr = valu_bwd_lds_dkdv(dkd, TV);
  // beyond the default dynamic-LDS limit (gfx950 has 160 KB per workgroup)
  (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&bwd_dq_valu_kernel<Tin>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lq);
  (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&bwd_dkdv_valu_kernel<Tin, false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lr);
  (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&bwd_dkdv_valu_kernel<Tin, true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lr);
  if (a.cslots) {  // time segments: local carries, combined in reverse
    Plan pc = p;
    pc.deal = 1;  // the carry pass skips every first segment
    const unsigned gc = xcd_grid(1, (long long)p.max_items * a.H, a.dv / TV);
    hipLaunchKernelGGL((bwd_dkdv_valu_kernel<Tin, true>), dim3(gc), dim3(256), lr, s,
                       (const Tin *)a.q, (const Tin *)a.k, (const Tin *)a.v,
                       (const Tin *)a.dout, a.ds_final, a.cslots, (Tin *)a.dv_out, a.ds0,
                       a.part_dk, pc, dec, a.scale, a.H, dkd, a.dv, TV);
    (void)launch_rcombine(p, a.ds_final, a.cslots, dec, a.H, dkd, a.dv, s);  // errors surface below
  }
  hipLaunchKernelGGL((bwd_dq_valu_kernel<Tin>), dim3(grid), dim3(256), lq, s,
                     (const Tin *)a.k, (const Tin *)a.v, (const Tin *)a.dout, a.s0, a.slots,
                     a.part_dq, p, dec, a.scale, a.H, dkd, a.dv, TV);
  hipLaunchKernelGGL((bwd_dkdv_valu_kernel<Tin, false>), dim3(grid), dim3(256), lr, s,
                     (const Tin *)a.q, (const Tin *)a.k, (const Tin *)a.v,
                     (const Tin *)a.dout, a.ds_final, a.cslots, (Tin *)a.dv_out, a.ds0,
                     a.part_dk, p, dec, a.scale, a.H, dkd, a.dv, TV);
  const long long n4 = (long long)p.total_T * a.H * (dkd / 4);
  hipLaunchKernelGGL((bwd_reduce_valu_kernel<Tin>), dim3((unsigned)((n4 + 255) / 256)),
                     dim3(256), 0, s, a.part_dq, a.part_dk, (Tin *)a.dq, (Tin *)a.dk,
                     (long long)p.total_T, a.H, dkd, a.dv / TV);
}

hipError_t launch_bwd_valu(int dt, const Plan &p, const BwdArgs &a, const Decay &dec,
                           hipStream_t s) {
  if (dt == 1) launch_bwd_valu_t<bf16>(p, a, dec, s);
  else launch_bwd_valu_t<float>(p, a, dec, s);
  return hipGetLastError();
}

}  // namespace gla
