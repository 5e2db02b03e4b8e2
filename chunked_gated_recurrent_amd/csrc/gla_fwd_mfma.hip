// gla_fwd_mfma.hip -- chunked Simple GLA forward for bf16 inputs with dk = 96
// (the Laplace head), 64 or 128 on the gfx950 matrix cores.
//
// A workgroup owns one (work item, head, dv tile) and walks the item's chunks
// in order; the fp32 state tile lives in MFMA accumulators for the whole
// walk. Per chunk of L <= 64 tokens (Laplace 3B / Trainium2 page, section
// "Challenge 1": chunk-internal masked linear attention plus the carried
// state, then a state advance by the decay accumulated over the chunk):
//     P^T[j][i] = (k_j . q_i) lambda^(i-j)   (j <= i, else 0)     K Q^T
//     O^T[c][i] = lambda^(i+1) (S^T Q^T)[c][i] + (V^T P^T)[c][i]
//     S[d][c]  <- lambda^L S[d][c] + (Ks^T V)[d][c],   Ks_j = lambda^(L-1-j) k_j
// All four products use v_mfma_f32_16x16x32_bf16 (fp32 accumulation).
//
// Roles. The output pass runs 8 waves: waves 0-3 ("output waves") own the 16
// output rows i = 16 w .. 16 w + 15 of every chunk, waves 4-7 ("state
// waves") own a 3 x 3 (or 3 x 2) block of state tiles. Wave w and wave w + 4
// share a SIMD, so each SIMD interleaves an output wave (42 MFMAs per chunk)
// with a state wave (18). The state waves publish the bf16 copy of S_c into
// one of two LDS buffers while the output waves read S_{c-1} from the other,
// so the roles meet only at the two barriers per chunk. The state-only pass
// (local end states of time segments) runs the state role alone on 4 waves.
//
// Data movement:
//   * global -> registers with raw buffer loads whose range is the chunk's
//     valid rows: rows past the end of a partial chunk (or every row of a
//     chunk past the end) read as zero without touching memory, and output
//     stores past the end are dropped. Loads run two chunks ahead in two
//     register stages, in straight-line code, so the compiler's memory
//     counter waits cover only the older stage;
//   * registers -> LDS, all tiles row-major (q, k, decay-scaled k, v);
//   * operands whose contraction index runs down the rows (v for both P V and
//     Ks^T V, Ks for Ks^T V) are read with ds_read_b64_tr_b16, the LDS
//     transpose read of gfx950: in each 16-lane group, lane i receives
//     element i % 4 of the 8-byte loads of lanes 4e + i / 4 (e = 0..3); when
//     lane s of the group loads row kb + s / 4, columns nb + 4 (s % 4) .. +3,
//     lane i receives rows kb .. kb+3 of column nb + i;
//   * outputs are staged through LDS (in the wave's own, already consumed
//     rows of the q tile) and written as 16-byte row segments.
//
// MFMA lane layout (lane l, l16 = l % 16, g = l / 16): A row l16 and B column
// l16 with the same 8 k-values for lane group g; D rows 4g..4g+3, column l16.
// The D layout of two P^T tiles (j blocks 2s, 2s+1) is exactly a B operand
// over the k-set {32s + 4g + r, 32s + 16 + 4g + r}, so P^T never leaves
// registers; the matching A operand (V^T) is read with the same k-set.
#include "gla_mfma.h"

namespace gla {

// ---------------------------------------------------------------------------
// Output role: 4 waves (role wave w owns rows 16 w .. 16 w + 15 of a chunk).
// ---------------------------------------------------------------------------
// GATE: the output gate y = o * act(g) is applied to each output value in
// fp32, before its single rounding to bf16; g is read from global memory in
// the output tiles' own layout (this lane's 4 columns of each column tile of
// its row), issued at the top of the chunk so it lands during the products.
template <int DVT, bool NORM, int DKT, bool GATE>
__device__ __forceinline__ void output_role(
    const bf16 *__restrict__ q, bf16 *__restrict__ o, const bf16 *__restrict__ gt, int gate,
    const Item &it, int h, int H, int dv, int c0, float scale, int rt, int w, bf16 *sQ,
    const bf16 *sK, const bf16 *sV, const bf16 *sSt0, const bf16 *sSt1,
    const float *sPow) {
  using M = MfCfg<DVT, DKT>;
  constexpr int C = M::C, DK = M::DK, QS = M::QS, VS = M::VS;
  constexpr int NCT = M::NCT, NKS = M::NKS, NJS = M::NJS, QV = M::QV;
  static_assert(DVT <= QS, "a wave stages its 16 x DVT output rows in its own q rows");
  const int lane = rt & 63, l16 = lane & 15, g = lane >> 4;
  const int tr_row = l16 >> 2, tr_col = 4 * (l16 & 3);
  const unsigned rowKb = (unsigned)(H * DK * 2), rowVb = (unsigned)(H * dv * 2);
  const int nch = (it.t1 - it.t0 + C - 1) / C;

  int rowQ[QV], colQ[QV];
#pragma unroll
  for (int m = 0; m < QV; ++m) {
    const int vi = rt + 256 * m;
    rowQ[m] = vi / M::NQV;
    colQ[m] = vi - rowQ[m] * M::NQV;
  }
  auto load_q = [&](int ch, u32x4(&r)[QV]) {
    const long long tb = (long long)it.t0 + (long long)ch * C;
    const __amdgpu_buffer_rsrc_t bq =
        buf_rsrc(q + (tb * H + h) * DK, (unsigned)chunk_rows(it, ch) * rowKb);
#pragma unroll
    for (int m = 0; m < QV; ++m)
      r[m] = __builtin_amdgcn_raw_buffer_load_b128(bq, rowQ[m] * rowKb + colQ[m] * 16, 0, 0);
  };
  constexpr int KBUF = C * QS, VBUF = C * VS;  // elements per chunk buffer
  auto store_q = [&](int buf, const u32x4(&r)[QV]) {
#pragma unroll
    for (int m = 0; m < QV; ++m)
      *reinterpret_cast<u32x4 *>(sQ + buf * KBUF + rowQ[m] * QS + 8 * colQ[m]) =
          NORM ? relu_bf16x8(r[m]) : r[m];
  };

  u32x4 ra[QV], rb[QV];
  load_q(0, ra);
  load_q(1, rb);
  __syncthreads();  // sPow ready
  const int i_row = 16 * w + l16;
  const float lam_i1 = sPow[i_row + 1];
  float maskw[4][4];  // causal decay mask of this lane's P^T column
#pragma unroll
  for (int J = 0; J < 4; ++J)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int diff = i_row - (16 * J + 4 * g + r);
      maskw[J][r] = diff >= 0 ? sPow[max(diff, 0)] : 0.f;
    }
  store_q(0, ra);

  auto body = [&](int ch, u32x4(&rnew)[QV], const u32x4(&rnext)[QV], const bf16 *st) {
    const long long tb = (long long)it.t0 + (long long)ch * C;
    const int L = chunk_rows(it, ch);
    const int cur = ch & 1;
    __syncthreads();  // chunk ch and S_{ch-1} are in LDS; chunk ch-1 is done
    load_q(ch + 2, rnew);
    store_q(cur ^ 1, rnext);
    u32x2 graw[NCT];  // GATE: g of this lane's outputs (rows past the end read 0)
    if (GATE) {
      const __amdgpu_buffer_rsrc_t bg =
          buf_rsrc(gt + tb * H * dv + (long long)h * dv + c0, (unsigned)L * rowVb);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
        graw[ct] = __builtin_amdgcn_raw_buffer_load_b64(
            bg, (unsigned)i_row * rowVb + (unsigned)(16 * ct + 4 * g) * 2, 0, 0);
    }
    const bf16 *cQ = sQ + cur * KBUF, *cK = sK + cur * KBUF, *cV = sV + cur * VBUF;
    bf16x8 qf[NKS];
#pragma unroll
    for (int s = 0; s < NKS; ++s)
      qf[s] = *reinterpret_cast<const bf16x8 *>(cQ + i_row * QS + 32 * s + 8 * g);
    // P^T tiles for j blocks 0..3 (tiles above the diagonal mask to zero)
    f32x4 p[4];
#pragma unroll
    for (int J = 0; J < 4; ++J) p[J] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NKS; ++s)
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(cK + (16 * J + l16) * QS + 32 * s + 8 * g);
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
        const bf16x8 sf = *reinterpret_cast<const bf16x8 *>(st + (16 * ct + l16) * QS + 32 * s + 8 * g);
        oacc[ct] = mfma(sf, qf[s], oacc[ct]);
      }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) oacc[ct] *= lam_i1;
#pragma unroll
    for (int s = 0; s < NJS; ++s)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const bf16 *base = cV + (32 * s + 4 * g + tr_row) * VS + 16 * ct + tr_col;
        const bf16x8 vf = cat8(tr4(base), tr4(base + 16 * VS));
        oacc[ct] = mfma(vf, pb[s], oacc[ct]);
      }
    // the output coefficient: scale, or for normalised linear attention
    // 1 / (phi(q_i) . z_i + eps) with the denominator formed like a 17th
    // column tile: z_{ch-1} (row DVT of the state buffer, the same row for
    // every lane) against Q^T, then a value tile of ones against P^T
    float coef = scale;
    if (NORM) {
      f32x4 den = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        const bf16x8 zf = *reinterpret_cast<const bf16x8 *>(st + DVT * QS + 32 * s + 8 * g);
        den = mfma(zf, qf[s], den);
      }
      den *= lam_i1;
      const bf16x8 ones = ones_bf16x8();
#pragma unroll
      for (int s = 0; s < NJS; ++s) den = mfma(ones, pb[s], den);
      // all four rows are equal; the hardware reciprocal (about 1 ulp) is
      // far below the bf16 rounding of the output
      coef = __builtin_amdgcn_rcpf(den[0] + kLinearAttnEps);
    }
    // stage the 16 x DVT output tile of this wave in its own rows of the
    // current q buffer (only this wave reads them, and qf is already loaded),
    // then write 16-byte row segments
    bf16 *so = sQ + cur * KBUF + 16 * w * QS;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      bf16x4 t;
      if (GATE) {
        const bf16x4 gv = __builtin_bit_cast(bf16x4, graw[ct]);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          t[r] = (bf16)(coef * oacc[ct][r] * gate_act((float)gv[r], gate));
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) t[r] = (bf16)(coef * oacc[ct][r]);
      }
      *reinterpret_cast<bf16x4 *>(so + l16 * QS + 16 * ct + 4 * g) = t;
    }
    const __amdgpu_buffer_rsrc_t bo =
        buf_rsrc(o + tb * H * dv + (long long)h * dv + c0, (unsigned)L * rowVb);
#pragma unroll
    for (int m = 0; m < M::OV; ++m) {
      const int vi = lane + 64 * m;
      const int row = vi / M::NVV, col = vi - (vi / M::NVV) * M::NVV;
      const u32x4 val = *reinterpret_cast<const u32x4 *>(so + row * QS + 8 * col);
      __builtin_amdgcn_raw_buffer_store_b128(val, bo, (16 * w + row) * rowVb + col * 16, 0, 0);
    }
  };
  for (int ch = 0; ch < nch; ch += 2) {  // a past-the-end chunk is all zeros
    body(ch, ra, rb, sSt1);               // reads S_{ch-1}
    body(ch + 1, rb, ra, sSt0);
  }
}

// ---------------------------------------------------------------------------
// kernels
// ---------------------------------------------------------------------------
template <int DVT, bool NORM, int DKT, bool GATE>
__global__ __launch_bounds__(512, 1) void fwd_out_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k,
    const bf16 *__restrict__ v, bf16 *__restrict__ o,
    const float *__restrict__ s0, float *__restrict__ s_final,
    float *__restrict__ slots, Plan plan, Decay dec, float scale, int H, int dv,
    int final_in_slot, NormPtrs np, const bf16 *__restrict__ gt, int gate) {
  using M = MfCfg<DVT, DKT>;
  // dk 128: the state waves scale k in registers (no third 64 x 144 tile),
  // which leaves LDS room for 64-column d_v tiles
  constexpr bool KSR = DKT == 128;
  __shared__ __attribute__((aligned(16))) bf16 sQ[2 * M::C * M::QS];
  __shared__ __attribute__((aligned(16))) bf16 sK[2 * M::C * M::QS];
  __shared__ __attribute__((aligned(16))) bf16 sKs[KSR ? 8 : 2 * M::C * M::QS];
  __shared__ __attribute__((aligned(16))) bf16 sV[2 * M::C * M::VS];
  __shared__ __attribute__((aligned(16))) bf16 sSt0[M::SROWS * M::QS];
  __shared__ __attribute__((aligned(16))) bf16 sSt1[M::SROWS * M::QS];
  __shared__ float sPow[M::C + 4];

  const int ndt = dv / DVT;
  int unit, dtile;
  xcd_unit(plan, ndt, plan.max_items * H, unit, dtile);
  if (unit >= plan.max_items * H) return;
  const int slot = unit / H;
  const int h = unit - slot * H;
  int idx;
  Item it;
  if (!slot_item(plan, slot, idx, it)) return;
  make_uniform(idx, it);
  const int tid = threadIdx.x;
  if (tid <= M::C) sPow[tid] = pow_f64(dec.lam[h], tid);
  const int role_wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c0 = dtile * DVT;
  if (role_wave < 4)
    output_role<DVT, NORM, DKT, GATE>(q, o, gt, gate, it, h, H, dv, c0, scale, tid & 255,
                                      role_wave, sQ, sK, sV, sSt0, sSt1, sPow);
  else
    state_role<DVT, true, NORM, DKT, KSR>(k, v, s0, s_final, slots, it, idx, h, H, dv, c0,
                                     final_in_slot, tid & 255, role_wave - 4, sK, sKs, sV,
                                     sSt0, sSt1, sPow, np);
}

template <int DVT, bool NORM, int DKT>
__global__ __launch_bounds__(256, 2) void fwd_state_kernel(
    const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    float *__restrict__ slots, Plan plan, Decay dec, int H, int dv, NormPtrs np) {
  using M = MfCfg<DVT, DKT>;
  __shared__ __attribute__((aligned(16))) bf16 sKs[2 * M::C * M::QS];
  __shared__ __attribute__((aligned(16))) bf16 sV[2 * M::C * M::VS];
  __shared__ float sPow[M::C + 4];

  const int ndt = dv / DVT;
  int unit, dtile;
  xcd_unit(plan, ndt, plan.max_items * H, unit, dtile);
  if (unit >= plan.max_items * H) return;
  const int slot = unit / H;
  const int h = unit - slot * H;
  int idx;
  Item it;
  if (!slot_item(plan, slot, idx, it)) return;
  make_uniform(idx, it);
  if (it.flags & kLastSeg) return;  // no later segment reads it
  const int tid = threadIdx.x;
  if (tid <= M::C) sPow[tid] = pow_f64(dec.lam[h], tid);
  // backward walk: it ends on the segment's first rows, where the output
  // pass starts next
  state_role<DVT, false, NORM, DKT, DKT == 128, true>(k, v, nullptr, nullptr, slots, it, idx,
                                                      h, H, dv,
                               dtile * DVT, 0, tid, __builtin_amdgcn_readfirstlane(tid >> 6),
                               nullptr, sKs, sV, nullptr, nullptr, sPow, np);
}

template <int DVT, bool NORM, int DKT>
static void launch_dvt(bool state_only, const Plan &p, const FwdArgs &a,
                       const Decay &dec, hipStream_t s) {
  const unsigned grid = xcd_grid(p.deal, (long long)p.max_items * a.H, a.dv / DVT);
  const NormPtrs np = {a.z0, a.z_final, a.zslots};
  if (state_only) {
    hipLaunchKernelGGL((fwd_state_kernel<DVT, NORM, DKT>), dim3(grid), dim3(256), 0, s,
                       (const bf16 *)a.k, (const bf16 *)a.v, a.slots, p, dec, a.H, a.dv, np);
    return;
  }
  if constexpr (!NORM) {  // the gated readout (the normalised attention has no gate)
    if (a.gate != kGateNone) {
      hipLaunchKernelGGL((fwd_out_kernel<DVT, false, DKT, true>), dim3(grid), dim3(512), 0, s,
                         (const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.v,
                         (bf16 *)a.o, a.s0, a.s_final, a.slots, p, dec, a.scale,
                         a.H, a.dv, a.final_in_slot, np, (const bf16 *)a.g, a.gate);
      return;
    }
  }
  hipLaunchKernelGGL((fwd_out_kernel<DVT, NORM, DKT, false>), dim3(grid), dim3(512), 0, s,
                     (const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.v,
                     (bf16 *)a.o, a.s0, a.s_final, a.slots, p, dec, a.scale,
                     a.H, a.dv, a.final_in_slot, np, (const bf16 *)nullptr, kGateNone);
}

// dk 96 runs d_v tiles of 96 or 64 columns, dk 64 tiles of 64 (a wave
// stages its output rows in its q rows, dk + 16 elements wide), dk 128
// tiles of 64 (with k scaled in registers: two double-buffered 64 x 128
// q/k tiles, 132 KB of LDS)
void launch_fwd_mfma(bool state_only, int dvt, const Plan &p, const FwdArgs &a,
                     const Decay &dec, hipStream_t s) {
  if (a.dk == 64) {
    if (a.norm) launch_dvt<64, true, 64>(state_only, p, a, dec, s);
    else launch_dvt<64, false, 64>(state_only, p, a, dec, s);
  } else if (a.dk == 128) {
    if (a.norm) launch_dvt<64, true, 128>(state_only, p, a, dec, s);
    else launch_dvt<64, false, 128>(state_only, p, a, dec, s);
  } else if (a.norm) {
    if (dvt == 96) launch_dvt<96, true, 96>(state_only, p, a, dec, s);
    else launch_dvt<64, true, 96>(state_only, p, a, dec, s);
  } else {
    if (dvt == 96) launch_dvt<96, false, 96>(state_only, p, a, dec, s);
    else launch_dvt<64, false, 96>(state_only, p, a, dec, s);
  }
}

}  // namespace gla
