// gla_fwd_mfma.hip -- chunked Simple GLA forward for bf16 inputs with dk = 96
// on the gfx950 matrix cores.
//
// One workgroup (4 waves) owns one (work item, head, dv tile) and walks the
// item's chunks in order; the fp32 state tile lives in MFMA accumulators for
// the whole walk. Per chunk of L <= 64 tokens (Laplace 3B / Trainium2 page,
// section "Challenge 1": chunk-internal masked linear attention plus the
// carried state, then a state advance by the decay accumulated over the
// chunk):
//     P^T[j][i] = (k_j . q_i) lambda^(i-j)   (j <= i, else 0)     K Q^T
//     O^T[c][i] = lambda^(i+1) (S^T Q^T)[c][i] + (V^T P^T)[c][i]
//     S[d][c]  <- lambda^L S[d][c] + (Ks^T V)[d][c],   Ks_j = lambda^(L-1-j) k_j
// All four products use v_mfma_f32_16x16x32_bf16 (fp32 accumulation).
//
// Data movement:
//   * global -> registers with raw buffer loads whose range is the chunk's
//     valid rows: rows past the end of a partial chunk read as zero and the
//     matching output stores are dropped, so there are no per-row branches;
//   * registers -> LDS, all tiles row-major (q, k, decay-scaled k, v) plus a
//     bf16 transposed copy of the state for the readout;
//   * operands whose contraction index runs down the rows (v for both P V and
//     Ks^T V, Ks for Ks^T V) are read with ds_read_b64_tr_b16, the LDS
//     transpose read of gfx950: in each 16-lane group, lane i receives
//     element i % 4 of the 8-byte loads of lanes 4e + i / 4 (e = 0..3); when
//     lane s of the group loads row kb + s / 4, columns nb + 4 (s % 4) .. +3,
//     lane i receives rows kb .. kb+3 of column nb + i.
//   * the next chunk's loads are issued before the current chunk's math.
//
// MFMA lane layout (lane l, l16 = l % 16, g = l / 16): A row l16 and B column
// l16 with the same 8 k-values for lane group g; D rows 4g..4g+3, column l16.
// The D layout of two P^T tiles (j blocks 2s, 2s+1) is exactly a B operand
// over the k-set {32s + 4g + r, 32s + 16 + 4g + r}, so P^T never leaves
// registers; the matching A operand (V^T) is read with the same k-set.
#include <stdlib.h>

#include "gla_device.h"

namespace gla {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Raw buffer resource (gfx9 family descriptor word 3) over `bytes` bytes.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *base,
                                                           unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0,
                                           (int)bytes, 0x00020000);
}

// Four bf16 of one column from four consecutive rows (see the header).
__device__ __forceinline__ bf16x4 tr4(const bf16 *p) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p);
  return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
  return (bf16x8){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int DVT, bool STATE_ONLY>
__global__ __launch_bounds__(256, 2) void fwd_mfma2_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k,
    const bf16 *__restrict__ v, bf16 *__restrict__ o,
    const float *__restrict__ s0, float *__restrict__ s_final,
    float *__restrict__ slots, Plan plan, Decay dec, float scale, int H, int dv,
    int final_in_slot) {
  constexpr int C = 64, DK = 96;
  constexpr int QS = DK + 8;     // LDS row stride of q, k, ks and S^T (elements)
  constexpr int VS = DVT + 8;    // LDS row stride of v
  constexpr int NCT = DVT / 16;  // 16-column tiles of the dv tile
  constexpr int NDT = DK / 16;   // 16-row tiles of dk
  constexpr int NKS = DK / 32;   // 32-deep steps over dk
  constexpr int NJS = C / 32;    // 32-deep steps over the chunk
  constexpr int SDT = NDT / 2, SCT = NCT / 2;  // state tiles per wave
  constexpr int NQV = DK / 8, NVV = DVT / 8;   // 16-byte vectors per row
  constexpr int QV = C * NQV / 256, VV = C * NVV / 256;
  static_assert(C * NQV % 256 == 0 && C * NVV % 256 == 0, "load split");
  static_assert(NCT % 2 == 0 && NDT % 2 == 0, "state split");

  __shared__ __attribute__((aligned(16))) bf16 sQ[STATE_ONLY ? 8 : C * QS];
  __shared__ __attribute__((aligned(16))) bf16 sK[STATE_ONLY ? 8 : C * QS];
  __shared__ __attribute__((aligned(16))) bf16 sKs[C * QS];
  __shared__ __attribute__((aligned(16))) bf16 sV[C * VS];
  __shared__ __attribute__((aligned(16))) bf16 sSt[STATE_ONLY ? 8 : DVT * QS];
  __shared__ float sPow[C + 4];

  const int ndt = dv / DVT;
  int unit, dtile;
  xcd_unit(ndt, unit, dtile);
  if (unit >= plan.max_items * H) return;
  const int idx = unit / H;
  const int h = unit - idx * H;
  Item it;
  if (!load_item(plan, idx, it)) return;
  if (STATE_ONLY && (it.flags & kLastSeg)) return;  // nothing reads it

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int c0 = dtile * DVT;
  const unsigned rowKb = (unsigned)(H * DK * 2);  // bytes between tokens, q/k
  const unsigned rowVb = (unsigned)(H * dv * 2);  // bytes between tokens, v/o
  const float lam = dec.lam[h];
  const int len = it.t1 - it.t0;
  const int nch = (len + C - 1) / C;

  if (tid <= C) sPow[tid] = pow_f64(lam, tid);

  // ---- state tiles of this wave: d tiles [dt0, dt0+SDT) x c tiles [ct0, ct0+SCT)
  const int dt0 = SDT * (w >> 1);
  const int ct0 = SCT * (w & 1);
  f32x4 accS[SDT][SCT];
  {
    const float *src = nullptr;
    if (!STATE_ONLY) {
      if (it.flags & kFirstSeg)
        src = s0 ? s0 + ((long long)it.n * H + h) * DK * dv : nullptr;
      else
        src = slots + ((long long)(idx - 1) * H + h) * DK * dv;
    }
#pragma unroll
    for (int a = 0; a < SDT; ++a)
#pragma unroll
      for (int b = 0; b < SCT; ++b) {
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
        if (src) {
          const int d = 16 * (dt0 + a) + 4 * g;
          const int c = c0 + 16 * (ct0 + b) + l16;
#pragma unroll
          for (int r = 0; r < 4; ++r) x[r] = src[(long long)(d + r) * dv + c];
        }
        accS[a][b] = x;
      }
  }

  // ---- per-thread load slots (same every chunk)
  int rowQ[QV], colQ[QV], rowV[VV], colV[VV];
#pragma unroll
  for (int m = 0; m < QV; ++m) {
    const int vi = tid + 256 * m;
    rowQ[m] = vi / NQV;
    colQ[m] = vi - rowQ[m] * NQV;
  }
#pragma unroll
  for (int m = 0; m < VV; ++m) {
    const int vi = tid + 256 * m;
    rowV[m] = vi / NVV;
    colV[m] = vi - rowV[m] * NVV;
  }
  u32x4 rq[QV], rk[QV], rv[VV];

  auto load_chunk = [&](int ch) {
    const int tb = it.t0 + ch * C;
    const int L = min(C, it.t1 - tb);
    const long long qk_off = ((long long)tb * H + h) * DK;
    const __amdgpu_buffer_rsrc_t bk = buf_rsrc(k + qk_off, (unsigned)L * rowKb);
    const __amdgpu_buffer_rsrc_t bv =
        buf_rsrc(v + (long long)tb * H * dv + (long long)h * dv + c0, (unsigned)L * rowVb);
    if (!STATE_ONLY) {
      const __amdgpu_buffer_rsrc_t bq = buf_rsrc(q + qk_off, (unsigned)L * rowKb);
#pragma unroll
      for (int m = 0; m < QV; ++m)
        rq[m] = __builtin_amdgcn_raw_buffer_load_b128(bq, rowQ[m] * rowKb + colQ[m] * 16, 0, 0);
    }
#pragma unroll
    for (int m = 0; m < QV; ++m)
      rk[m] = __builtin_amdgcn_raw_buffer_load_b128(bk, rowQ[m] * rowKb + colQ[m] * 16, 0, 0);
#pragma unroll
    for (int m = 0; m < VV; ++m)
      rv[m] = __builtin_amdgcn_raw_buffer_load_b128(bv, rowV[m] * rowVb + colV[m] * 16, 0, 0);
  };

  auto store_chunk = [&](int L) {
#pragma unroll
    for (int m = 0; m < QV; ++m) {
      const int r = rowQ[m];
      if (!STATE_ONLY) {
        *reinterpret_cast<u32x4 *>(sQ + r * QS + 8 * colQ[m]) = rq[m];
        *reinterpret_cast<u32x4 *>(sK + r * QS + 8 * colQ[m]) = rk[m];
      }
      // decay-scaled copy: lambda^(L-1-r) k_r (rows past the end are zero)
      const float wgt = r < L ? sPow[max(L - 1 - r, 0)] : 0.f;
      const bf16x8 kv = __builtin_bit_cast(bf16x8, rk[m]);
      bf16x8 ks;
#pragma unroll
      for (int e = 0; e < 8; ++e) ks[e] = (bf16)((float)kv[e] * wgt);
      *reinterpret_cast<bf16x8 *>(sKs + r * QS + 8 * colQ[m]) = ks;
    }
#pragma unroll
    for (int m = 0; m < VV; ++m)
      *reinterpret_cast<u32x4 *>(sV + rowV[m] * VS + 8 * colV[m]) = rv[m];
  };

  auto store_state_lds = [&]() {
#pragma unroll
    for (int a = 0; a < SDT; ++a)
#pragma unroll
      for (int b = 0; b < SCT; ++b) {
        bf16x4 t;
#pragma unroll
        for (int r = 0; r < 4; ++r) t[r] = (bf16)accS[a][b][r];
        const int c = 16 * (ct0 + b) + l16;
        *reinterpret_cast<bf16x4 *>(sSt + c * QS + 16 * (dt0 + a) + 4 * g) = t;
      }
  };

  if (nch > 0) load_chunk(0);
  __syncthreads();  // sPow ready

  // per-lane constants: output row i = 16 w + l16 of every chunk, its
  // lambda^(i+1), and the causal decay mask of its P^T column
  const int i_row = 16 * w + l16;
  const float lam_i1 = sPow[i_row + 1];
  float maskw[4][4];
#pragma unroll
  for (int J = 0; J < 4; ++J)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int diff = i_row - (16 * J + 4 * g + r);
      maskw[J][r] = diff >= 0 ? sPow[max(diff, 0)] : 0.f;
    }
  // transpose-read lane offsets
  const int tr_row = l16 >> 2, tr_col = 4 * (l16 & 3);

  if (nch > 0) {
    store_chunk(min(C, len));
    if (!STATE_ONLY) store_state_lds();
  }
  __syncthreads();

  for (int ch = 0; ch < nch; ++ch) {
    const int tb = it.t0 + ch * C;
    const int L = min(C, it.t1 - tb);
    if (ch + 1 < nch) load_chunk(ch + 1);

    if (!STATE_ONLY) {
      bf16x8 qf[NKS];
#pragma unroll
      for (int s = 0; s < NKS; ++s)
        qf[s] = *reinterpret_cast<const bf16x8 *>(sQ + i_row * QS + 32 * s + 8 * g);

      // P^T tiles for j blocks 0..3 (tiles above the diagonal mask to zero)
      f32x4 p[4];
#pragma unroll
      for (int J = 0; J < 4; ++J) p[J] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NKS; ++s)
#pragma unroll
        for (int J = 0; J < 4; ++J) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(sK + (16 * J + l16) * QS + 32 * s + 8 * g);
          p[J] = mfma(kf, qf[s], p[J]);
        }
      bf16x8 pb[NJS];
#pragma unroll
      for (int s = 0; s < NJS; ++s)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pb[s][r] = (bf16)(p[2 * s][r] * maskw[2 * s][r]);
          pb[s][4 + r] = (bf16)(p[2 * s + 1][r] * maskw[2 * s + 1][r]);
        }

      // O^T = lambda^(i+1) S^T Q^T + V^T P^T for all c tiles
      f32x4 oacc[NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) oacc[ct] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NKS; ++s)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const bf16x8 sf = *reinterpret_cast<const bf16x8 *>(sSt + (16 * ct + l16) * QS + 32 * s + 8 * g);
          oacc[ct] = mfma(sf, qf[s], oacc[ct]);
        }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) oacc[ct] *= lam_i1;
#pragma unroll
      for (int s = 0; s < NJS; ++s)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const bf16 *base = sV + (32 * s + 4 * g + tr_row) * VS + 16 * ct + tr_col;
          const bf16x8 vf = cat8(tr4(base), tr4(base + 16 * VS));
          oacc[ct] = mfma(vf, pb[s], oacc[ct]);
        }
      const __amdgpu_buffer_rsrc_t bo =
          buf_rsrc(o + (long long)tb * H * dv + (long long)h * dv + c0, (unsigned)L * rowVb);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        bf16x4 t;
#pragma unroll
        for (int r = 0; r < 4; ++r) t[r] = (bf16)(scale * oacc[ct][r]);
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, t), bo,
                                              i_row * rowVb + (16 * ct + 4 * g) * 2, 0, 0);
      }
    }

    // S <- lambda^L S + Ks^T V   (k-set {32s + 8g .. 32s + 8g + 7})
    {
      const float lamL = sPow[L];
#pragma unroll
      for (int a = 0; a < SDT; ++a)
#pragma unroll
        for (int b = 0; b < SCT; ++b) accS[a][b] *= lamL;
#pragma unroll
      for (int s = 0; s < NJS; ++s) {
        bf16x8 af[SDT], bfr[SCT];
        const int row = 32 * s + 8 * g + tr_row;
#pragma unroll
        for (int a = 0; a < SDT; ++a) {
          const bf16 *base = sKs + row * QS + 16 * (dt0 + a) + tr_col;
          af[a] = cat8(tr4(base), tr4(base + 4 * QS));
        }
#pragma unroll
        for (int b = 0; b < SCT; ++b) {
          const bf16 *base = sV + row * VS + 16 * (ct0 + b) + tr_col;
          bfr[b] = cat8(tr4(base), tr4(base + 4 * VS));
        }
#pragma unroll
        for (int a = 0; a < SDT; ++a)
#pragma unroll
          for (int b = 0; b < SCT; ++b) accS[a][b] = mfma(af[a], bfr[b], accS[a][b]);
      }
    }

    __syncthreads();  // all waves are done with this chunk's tiles
    if (ch + 1 < nch) {
      store_chunk(min(C, it.t1 - (tb + C)));
      if (!STATE_ONLY) store_state_lds();
    }
    __syncthreads();
  }

  // ---- final state: local end state to its slot, or the sequence's final
  float *dst = nullptr;
  if (STATE_ONLY || ((it.flags & kLastSeg) && final_in_slot))
    dst = slots + ((long long)idx * H + h) * DK * dv;
  else if ((it.flags & kLastSeg) && s_final)
    dst = s_final + ((long long)it.n * H + h) * DK * dv;
  if (dst) {
#pragma unroll
    for (int a = 0; a < SDT; ++a)
#pragma unroll
      for (int b = 0; b < SCT; ++b) {
        const int d = 16 * (dt0 + a) + 4 * g;
        const int c = c0 + 16 * (ct0 + b) + l16;
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(long long)(d + r) * dv + c] = accS[a][b][r];
      }
  }
}

// ---------------------------------------------------------------------------
// Output pass with split roles (8 waves)
// ---------------------------------------------------------------------------
// Waves 0-3 ("output waves") own the 16 output rows i = 16 w .. 16 w + 15 of
// every chunk; waves 4-7 ("state waves") own a 3 x 3 (or 3 x 2) block of
// state tiles and advance the state. Wave w and wave w + 4 share a SIMD, so
// each SIMD interleaves an output wave (42 MFMAs per chunk) with a state
// wave (18). The state waves write the bf16 copy of S_c into one of two
// buffers while the output waves read S_{c-1} from the other, so the roles
// only meet at the two barriers per chunk. Global loads run two chunks ahead
// in registers (q by the output waves, k and v by the state waves). Outputs
// are staged through a per-wave LDS tile and written as 16-byte row segments.
template <int DVT>
__global__ __launch_bounds__(512, 1) void fwd_mfma3_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k,
    const bf16 *__restrict__ v, bf16 *__restrict__ o,
    const float *__restrict__ s0, float *__restrict__ s_final,
    float *__restrict__ slots, Plan plan, Decay dec, float scale, int H, int dv,
    int final_in_slot) {
  constexpr int C = 64, DK = 96;
  constexpr int QS = DK + 8, VS = DVT + 8;
  constexpr int NCT = DVT / 16, NDT = DK / 16, NKS = DK / 32, NJS = C / 32;
  constexpr int SDT = NDT / 2, SCT = NCT / 2;
  constexpr int NQV = DK / 8, NVV = DVT / 8;
  constexpr int QV = C * NQV / 256;   // 16-byte q (or k) vectors per thread of a role
  constexpr int VV = C * NVV / 256;   // 16-byte v vectors per state thread
  constexpr int OV = 16 * NVV / 64;   // 16-byte output vectors per output lane
  static_assert(C * NQV % 256 == 0 && C * NVV % 256 == 0 && 16 * NVV % 64 == 0, "split");

  __shared__ __attribute__((aligned(16))) bf16 sQ[C * QS];
  __shared__ __attribute__((aligned(16))) bf16 sK[C * QS];
  __shared__ __attribute__((aligned(16))) bf16 sKs[C * QS];
  __shared__ __attribute__((aligned(16))) bf16 sV[C * VS];
  __shared__ __attribute__((aligned(16))) bf16 sSt[2][DVT * QS];
  __shared__ __attribute__((aligned(16))) bf16 sO[4][16 * VS];
  __shared__ float sPow[C + 4];

  const int ndt = dv / DVT;
  int unit, dtile;
  xcd_unit(ndt, unit, dtile);
  if (unit >= plan.max_items * H) return;
  const int idx = unit / H;
  const int h = unit - idx * H;
  Item it;
  if (!load_item(plan, idx, it)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w8 = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool out_role = w8 < 4;
  const int w = w8 & 3;
  const int rt = tid & 255;  // thread index within the role
  const int l16 = lane & 15, g = lane >> 4;
  const int c0 = dtile * DVT;
  const unsigned rowKb = (unsigned)(H * DK * 2);
  const unsigned rowVb = (unsigned)(H * dv * 2);
  const float lam = dec.lam[h];
  const int len = it.t1 - it.t0;
  const int nch = (len + C - 1) / C;
  const int tr_row = l16 >> 2, tr_col = 4 * (l16 & 3);
  auto chunk_len = [&](int ch) { return min(C, it.t1 - (it.t0 + ch * C)); };

  if (tid <= C) sPow[tid] = pow_f64(lam, tid);

  if (out_role) {
    // ======================= output waves =======================
    int rowQ[QV], colQ[QV];
#pragma unroll
    for (int m = 0; m < QV; ++m) {
      const int vi = rt + 256 * m;
      rowQ[m] = vi / NQV;
      colQ[m] = vi - rowQ[m] * NQV;
    }
    u32x4 ra[QV], rb[QV];
    auto load_q = [&](int ch, u32x4 (&r)[QV]) {
      const int tb = it.t0 + ch * C;
      const __amdgpu_buffer_rsrc_t bq =
          buf_rsrc(q + ((long long)tb * H + h) * DK, (unsigned)chunk_len(ch) * rowKb);
#pragma unroll
      for (int m = 0; m < QV; ++m)
        r[m] = __builtin_amdgcn_raw_buffer_load_b128(bq, rowQ[m] * rowKb + colQ[m] * 16, 0, 0);
    };
    auto store_q = [&](const u32x4 (&r)[QV]) {
#pragma unroll
      for (int m = 0; m < QV; ++m)
        *reinterpret_cast<u32x4 *>(sQ + rowQ[m] * QS + 8 * colQ[m]) = r[m];
    };
    if (nch > 0) load_q(0, ra);
    if (nch > 1) load_q(1, rb);
    __syncthreads();  // sPow ready
    const int i_row = 16 * w + l16;
    const float lam_i1 = sPow[i_row + 1];
    float maskw[4][4];
#pragma unroll
    for (int J = 0; J < 4; ++J)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int diff = i_row - (16 * J + 4 * g + r);
        maskw[J][r] = diff >= 0 ? sPow[max(diff, 0)] : 0.f;
      }
    if (nch > 0) store_q(ra);
    __syncthreads();

    auto body = [&](int ch, u32x4 (&rnew)[QV], const u32x4 (&rnext)[QV]) {
      const int tb = it.t0 + ch * C;
      const int L = chunk_len(ch);
      if (ch + 2 < nch) load_q(ch + 2, rnew);
      const bf16 *st = sSt[(ch + 1) & 1];  // S_{ch-1}
      bf16x8 qf[NKS];
#pragma unroll
      for (int s = 0; s < NKS; ++s)
        qf[s] = *reinterpret_cast<const bf16x8 *>(sQ + i_row * QS + 32 * s + 8 * g);
      f32x4 p[4];
#pragma unroll
      for (int J = 0; J < 4; ++J) p[J] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NKS; ++s)
#pragma unroll
        for (int J = 0; J < 4; ++J) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(sK + (16 * J + l16) * QS + 32 * s + 8 * g);
          p[J] = mfma(kf, qf[s], p[J]);
        }
      bf16x8 pb[NJS];
#pragma unroll
      for (int s = 0; s < NJS; ++s)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pb[s][r] = (bf16)(p[2 * s][r] * maskw[2 * s][r]);
          pb[s][4 + r] = (bf16)(p[2 * s + 1][r] * maskw[2 * s + 1][r]);
        }
      f32x4 oacc[NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) oacc[ct] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NKS; ++s)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const bf16x8 sf = *reinterpret_cast<const bf16x8 *>(st + (16 * ct + l16) * QS + 32 * s + 8 * g);
          oacc[ct] = mfma(sf, qf[s], oacc[ct]);
        }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) oacc[ct] *= lam_i1;
#pragma unroll
      for (int s = 0; s < NJS; ++s)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const bf16 *base = sV + (32 * s + 4 * g + tr_row) * VS + 16 * ct + tr_col;
          const bf16x8 vf = cat8(tr4(base), tr4(base + 16 * VS));
          oacc[ct] = mfma(vf, pb[s], oacc[ct]);
        }
      // stage the 16 x DVT output tile of this wave, then 16-byte row stores
      bf16 *so = sO[w];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        bf16x4 t;
#pragma unroll
        for (int r = 0; r < 4; ++r) t[r] = (bf16)(scale * oacc[ct][r]);
        *reinterpret_cast<bf16x4 *>(so + l16 * VS + 16 * ct + 4 * g) = t;
      }
      const __amdgpu_buffer_rsrc_t bo =
          buf_rsrc(o + (long long)tb * H * dv + (long long)h * dv + c0, (unsigned)L * rowVb);
#pragma unroll
      for (int m = 0; m < OV; ++m) {
        const int vi = lane + 64 * m;
        const int row = vi / NVV, col = vi - (vi / NVV) * NVV;
        const u32x4 val = *reinterpret_cast<const u32x4 *>(so + row * VS + 8 * col);
        __builtin_amdgcn_raw_buffer_store_b128(val, bo, (16 * w + row) * rowVb + col * 16, 0, 0);
      }
      __syncthreads();  // everyone is done with chunk ch
      if (ch + 1 < nch) store_q(rnext);
      __syncthreads();
    };
    for (int ch = 0; ch < nch; ch += 2) {
      body(ch, ra, rb);
      if (ch + 1 < nch) body(ch + 1, rb, ra);
    }
  } else {
    // ======================= state waves =======================
    const int dt0 = SDT * (w >> 1);
    const int ct0 = SCT * (w & 1);
    f32x4 accS[SDT][SCT];
    {
      const float *src;
      if (it.flags & kFirstSeg)
        src = s0 ? s0 + ((long long)it.n * H + h) * DK * dv : nullptr;
      else
        src = slots + ((long long)(idx - 1) * H + h) * DK * dv;
#pragma unroll
      for (int a = 0; a < SDT; ++a)
#pragma unroll
        for (int b = 0; b < SCT; ++b) {
          f32x4 x = {0.f, 0.f, 0.f, 0.f};
          if (src) {
            const int d = 16 * (dt0 + a) + 4 * g;
            const int c = c0 + 16 * (ct0 + b) + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) x[r] = src[(long long)(d + r) * dv + c];
          }
          accS[a][b] = x;
        }
    }
    int rowK[QV], colK[QV], rowV[VV], colV[VV];
#pragma unroll
    for (int m = 0; m < QV; ++m) {
      const int vi = rt + 256 * m;
      rowK[m] = vi / NQV;
      colK[m] = vi - rowK[m] * NQV;
    }
#pragma unroll
    for (int m = 0; m < VV; ++m) {
      const int vi = rt + 256 * m;
      rowV[m] = vi / NVV;
      colV[m] = vi - rowV[m] * NVV;
    }
    u32x4 ka[QV], kb[QV], va[VV], vb[VV];
    auto load_kv = [&](int ch, u32x4 (&rk)[QV], u32x4 (&rv)[VV]) {
      const int tb = it.t0 + ch * C;
      const unsigned L = (unsigned)chunk_len(ch);
      const __amdgpu_buffer_rsrc_t bk = buf_rsrc(k + ((long long)tb * H + h) * DK, L * rowKb);
      const __amdgpu_buffer_rsrc_t bv =
          buf_rsrc(v + (long long)tb * H * dv + (long long)h * dv + c0, L * rowVb);
#pragma unroll
      for (int m = 0; m < QV; ++m)
        rk[m] = __builtin_amdgcn_raw_buffer_load_b128(bk, rowK[m] * rowKb + colK[m] * 16, 0, 0);
#pragma unroll
      for (int m = 0; m < VV; ++m)
        rv[m] = __builtin_amdgcn_raw_buffer_load_b128(bv, rowV[m] * rowVb + colV[m] * 16, 0, 0);
    };
    auto store_kv = [&](int L, const u32x4 (&rk)[QV], const u32x4 (&rv)[VV]) {
#pragma unroll
      for (int m = 0; m < QV; ++m) {
        const int r = rowK[m];
        *reinterpret_cast<u32x4 *>(sK + r * QS + 8 * colK[m]) = rk[m];
        const float wgt = r < L ? sPow[max(L - 1 - r, 0)] : 0.f;
        const bf16x8 kv = __builtin_bit_cast(bf16x8, rk[m]);
        bf16x8 ks;
#pragma unroll
        for (int e = 0; e < 8; ++e) ks[e] = (bf16)((float)kv[e] * wgt);
        *reinterpret_cast<bf16x8 *>(sKs + r * QS + 8 * colK[m]) = ks;
      }
#pragma unroll
      for (int m = 0; m < VV; ++m)
        *reinterpret_cast<u32x4 *>(sV + rowV[m] * VS + 8 * colV[m]) = rv[m];
    };
    auto store_state = [&](bf16 *dst) {
#pragma unroll
      for (int a = 0; a < SDT; ++a)
#pragma unroll
        for (int b = 0; b < SCT; ++b) {
          bf16x4 t;
#pragma unroll
          for (int r = 0; r < 4; ++r) t[r] = (bf16)accS[a][b][r];
          const int c = 16 * (ct0 + b) + l16;
          *reinterpret_cast<bf16x4 *>(dst + c * QS + 16 * (dt0 + a) + 4 * g) = t;
        }
    };
    if (nch > 0) load_kv(0, ka, va);
    if (nch > 1) load_kv(1, kb, vb);
    __syncthreads();  // sPow ready
    if (nch > 0) store_kv(chunk_len(0), ka, va);
    store_state(sSt[1]);  // S_{-1}: the incoming state
    __syncthreads();

    auto body = [&](int ch, u32x4 (&rkn)[QV], u32x4 (&rvn)[VV],
                    const u32x4 (&rkx)[QV], const u32x4 (&rvx)[VV]) {
      const int L = chunk_len(ch);
      if (ch + 2 < nch) load_kv(ch + 2, rkn, rvn);
      const float lamL = sPow[L];
#pragma unroll
      for (int a = 0; a < SDT; ++a)
#pragma unroll
        for (int b = 0; b < SCT; ++b) accS[a][b] *= lamL;
#pragma unroll
      for (int s = 0; s < NJS; ++s) {
        bf16x8 af[SDT], bfr[SCT];
        const int row = 32 * s + 8 * g + tr_row;
#pragma unroll
        for (int a = 0; a < SDT; ++a) {
          const bf16 *base = sKs + row * QS + 16 * (dt0 + a) + tr_col;
          af[a] = cat8(tr4(base), tr4(base + 4 * QS));
        }
#pragma unroll
        for (int b = 0; b < SCT; ++b) {
          const bf16 *base = sV + row * VS + 16 * (ct0 + b) + tr_col;
          bfr[b] = cat8(tr4(base), tr4(base + 4 * VS));
        }
#pragma unroll
        for (int a = 0; a < SDT; ++a)
#pragma unroll
          for (int b = 0; b < SCT; ++b) accS[a][b] = mfma(af[a], bfr[b], accS[a][b]);
      }
      store_state(sSt[ch & 1]);  // S_ch for the next chunk's readout
      __syncthreads();
      if (ch + 1 < nch) store_kv(chunk_len(ch + 1), rkx, rvx);
      __syncthreads();
    };
    for (int ch = 0; ch < nch; ch += 2) {
      body(ch, ka, va, kb, vb);
      if (ch + 1 < nch) body(ch + 1, kb, vb, ka, va);
    }

    float *dst = nullptr;
    if ((it.flags & kLastSeg) && final_in_slot)
      dst = slots + ((long long)idx * H + h) * DK * dv;
    else if ((it.flags & kLastSeg) && s_final)
      dst = s_final + ((long long)it.n * H + h) * DK * dv;
    if (dst) {
#pragma unroll
      for (int a = 0; a < SDT; ++a)
#pragma unroll
        for (int b = 0; b < SCT; ++b) {
          const int d = 16 * (dt0 + a) + 4 * g;
          const int c = c0 + 16 * (ct0 + b) + l16;
#pragma unroll
          for (int r = 0; r < 4; ++r) dst[(long long)(d + r) * dv + c] = accS[a][b][r];
        }
    }
  }
}

template <int DVT>
static void launch3(const Plan &p, const FwdArgs &a, const Decay &dec, hipStream_t s) {
  const int ndt = a.dv / DVT;
  const unsigned grid = xcd_grid((long long)p.max_items * a.H, ndt);
  hipLaunchKernelGGL((fwd_mfma3_kernel<DVT>), dim3(grid), dim3(512), 0, s,
                     (const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.v,
                     (bf16 *)a.o, a.s0, a.s_final, a.slots, p, dec, a.scale,
                     a.H, a.dv, a.final_in_slot);
}

template <int DVT, bool SO>
static void launch2(const Plan &p, const FwdArgs &a, const Decay &dec,
                    hipStream_t s) {
  const int ndt = a.dv / DVT;
  const unsigned grid = xcd_grid((long long)p.max_items * a.H, ndt);
  hipLaunchKernelGGL((fwd_mfma2_kernel<DVT, SO>), dim3(grid), dim3(256), 0, s,
                     (const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.v,
                     (bf16 *)a.o, a.s0, a.s_final, a.slots, p, dec, a.scale,
                     a.H, a.dv, a.final_in_slot);
}

void launch_fwd_mfma2(bool state_only, int dvt, const Plan &p, const FwdArgs &a,
                      const Decay &dec, hipStream_t s) {
  if (!state_only && !getenv("GLA_FWD_V2")) {
    if (dvt == 96) launch3<96>(p, a, dec, s);
    else launch3<64>(p, a, dec, s);
    return;
  }
  if (dvt == 96) {
    if (state_only) launch2<96, true>(p, a, dec, s);
    else launch2<96, false>(p, a, dec, s);
  } else {
    if (state_only) launch2<64, true>(p, a, dec, s);
    else launch2<64, false>(p, a, dec, s);
  }
}

}  // namespace gla
