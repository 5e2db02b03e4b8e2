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
  state_role<DVT, false, NORM, DKT, DKT == 128, true>(
      k, v, nullptr, nullptr, slots, it, idx, h, H, dv, dtile * DVT, 0, tid,
      __builtin_amdgcn_readfirstlane(tid >> 6), nullptr, sKs, sV, nullptr, nullptr, sPow, np);
}

// ---------------------------------------------------------------------------
// Long sequences in one launch: the chained scan
// ---------------------------------------------------------------------------
// The segmented forward as one pass over the segments (Laplace 3B /
// Trainium2 page, "Challenge 1": only the state chain between chunks is
// sequential; states compose as affine maps, [RecFree] section 3.2). The
// workgroup of (item i, head, d_v tile):
//   1. unless i is its sequence's last item: forms the item's local end
//      state U_i (waves 0-3 over the first half of its chunks, waves 4-7 over
//      the rest; U_i = lambda^(len of the rest) U_first + U_rest), writes it
//      to its slot and raises its flag to 1;
//   2. forms its incoming state S_in(i): s0 for a sequence's first item,
//      else by looking back over the items before it, nearest first: an
//      item whose flag is 2 has published S after it (its inclusive state)
//      and ends the look-back; an item at flag 1 contributes its U and the
//      look-back goes on (past the first item, s0 ends it):
//      S_in(i) = sum over the terms of lambda^(t0_i - end of term) x term.
//      Unless i is last, it then publishes its own inclusive state
//      lambda^(len i) S_in(i) + U_i and raises its flag to 2;
//   3. runs the output walk from S_in(i), as fwd_out_kernel.
// Workgroup ids run item-major, and a workgroup only waits on items before
// its own in the same sequence, i.e. on smaller ids; the dispatcher hands
// out each XCD's workgroups in id order and step 1 never waits, so every
// awaited flag is raised whether or not the grid fits the GPU at once. Each
// wait is still bounded (about a second of wall clock); a workgroup that
// gives up fills its S_in with NaN, so the failure shows in every output of
// its item instead of passing silently.
// Within an item's id block the units are dealt to the XCDs by chain_unit.
// It is the library's second scheme for long sequences, selected with
// GLA_FWD_CHAIN=1; the three launches stay the default because they measured
// faster (one 65,536-token sequence, 16 heads: 369 against 493 us per call).
// Timestamps taken inside a copy of this kernel put the difference in three
// places: the local states end at 127-168 us against 123 us for the state
// pass (two half-walks per workgroup, and the last items' workgroups idle);
// the look-back costs 20-70 us, one memory round trip per term while every
// other workgroup streams; and the output walks then start up to 80 us
// apart, so the d_v tiles of a head no longer read their q and k rows
// together (270-300 us against 242 us for the output pass).
// Workspace (each [max_items][H][dk][dv] fp32 but the flags): slots (U_i),
// incl (inclusive states), sin (S_in(i) at sin[i-1], the layout the output
// walk reads; sin[i] is the second half-walk's scratch until item i+1
// writes it) and flags [max_items][H][d_v tiles], zeroed before the launch.
constexpr int kChainMaxItems = 256;  // items of one sequence (look-back table)

template <int DVT, int DKT, bool GATE>
__global__ __launch_bounds__(512, 1) void fwd_chain_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    bf16 *__restrict__ o, const float *__restrict__ s0, float *__restrict__ s_final,
    float *__restrict__ slots, float *__restrict__ incl, float *__restrict__ sin,
    int *__restrict__ flags, Plan plan, Decay dec, float scale, int H, int dv,
    int final_in_slot, const bf16 *__restrict__ gt, int gate) {
  using M = MfCfg<DVT, DKT>;
  // d_k 128 keeps the three-launch path: its output walk scales k in
  // registers to fit the LDS, which leaves no room for the second half-walk
  static_assert(DKT != 128, "the chained scan takes d_k 64 and 96");
  static_assert(M::VS <= M::QS, "the second half-walk keeps its v tiles in sK");
  constexpr bool KSR = false;
  __shared__ __attribute__((aligned(16))) bf16 sQ[2 * M::C * M::QS];
  __shared__ __attribute__((aligned(16))) bf16 sK[2 * M::C * M::QS];
  __shared__ __attribute__((aligned(16))) bf16 sKs[2 * M::C * M::QS];
  __shared__ __attribute__((aligned(16))) bf16 sV[2 * M::C * M::VS];
  __shared__ __attribute__((aligned(16))) bf16 sSt0[M::SROWS * M::QS];
  __shared__ __attribute__((aligned(16))) bf16 sSt1[M::SROWS * M::QS];
  __shared__ float sPow[M::C + 4];
  // look-back terms: j >= 0 is U_j, -1 - j the inclusive state of item j,
  // kS0Term the sequence's s0; sA their decays
  constexpr int kS0Term = -0x40000000;
  __shared__ int sTerm[kChainMaxItems + 1];
  __shared__ float sA[kChainMaxItems + 1];
  __shared__ int sN, sFail;

  const int ndt = dv / DVT;
  const int U = H * ndt;  // workgroups per item (H is a multiple of 8)
  const int idx = (int)blockIdx.x / U;
  int h, dtile;
  chain_unit((int)blockIdx.x - idx * U, U, ndt, h, dtile);
  const int su = h * ndt + dtile;  // this unit's flag within the item
  Item it;
  if (!load_item(plan, idx, it)) return;
  int idx_u = idx;
  make_uniform(idx_u, it);
  const int tid = threadIdx.x;
  if (tid <= M::C) sPow[tid] = pow_f64(dec.lam[h], tid);
  const int role_wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c0 = dtile * DVT;
  const long long item_stride = (long long)H * DKT * dv;
  const long long tile_off = (long long)h * DKT * dv + c0;  // this tile within a slot
  constexpr int NE = DKT * DVT;  // state elements of the tile
  int *flag = flags + (long long)idx * U + su;
  const bool last = (it.flags & kLastSeg) != 0, first = (it.flags & kFirstSeg) != 0;

  // 1. local end state
  if (!last) {
    const int nch = (it.t1 - it.t0 + M::C - 1) / M::C;
    const int nA = (nch + 1) >> 1;
    const int niter = (nA + 1) & ~1;  // both halves pass the same barriers
    const int tm = min(it.t0 + nA * M::C, it.t1);
    Item part = it;
    if (role_wave < 4) {
      part.t1 = tm;
      state_role<DVT, false, false, DKT, KSR, true>(k, v, nullptr, nullptr, slots, part, idx,
                                                    h, H, dv, c0, 0, tid, role_wave, nullptr,
                                                    sKs, sV, nullptr, nullptr, sPow,
                                                    NormPtrs{}, niter);
    } else {
      part.t0 = tm;
      state_role<DVT, false, false, DKT, KSR, true>(k, v, nullptr, nullptr, sin, part, idx,
                                                    h, H, dv, c0, 0, tid & 255,
                                                    role_wave - 4, nullptr, sQ, sK, nullptr,
                                                    nullptr, sPow, NormPtrs{}, niter);
    }
    __syncthreads();  // both half states are written
    const float aB = pow_f64(dec.lam[h], it.t1 - tm);
    float *ua = slots + (long long)idx * item_stride + tile_off;
    const float *ub = sin + (long long)idx * item_stride + tile_off;
    for (int e = tid; e < NE; e += 512) {
      const long long off = (long long)(e / DVT) * dv + (e % DVT);
      ua[off] = fmaf(aB, ua[off], ub[off]);
    }
    // every thread's stores reach the device-coherent level before the flag
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (tid == 0) __hip_atomic_store(flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // 2. incoming state; inclusive state published
  if (tid == 0) {
    int n = 0, fail = 0;
    if (first) {
      sTerm[n] = kS0Term;
      sA[n++] = 1.0f;
    } else {
      int seq_first, seq_last;
      seq_items(plan, it.n, seq_first, seq_last);
      const unsigned long long t_start = wall_clock64();
      const unsigned long long limit = 100000000ull;  // 1 s of the 100 MHz wall clock
      for (int j = idx - 1;; --j) {
        if (j < seq_first || n == kChainMaxItems) {  // (the host keeps n below the cap)
          Item f0 = {0, it.t0, it.t0, 0};
          load_item(plan, seq_first, f0);
          sTerm[n] = kS0Term;
          sA[n++] = pow_f64(dec.lam[h], it.t0 - f0.t0);
          break;
        }
        const int *fj = flags + (long long)j * U + su;
        int fv;
        while ((fv = __hip_atomic_load(fj, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) == 0) {
          if ((unsigned long long)wall_clock64() - t_start > limit) {
            fail = 1;
            break;
          }
          __builtin_amdgcn_s_sleep(2);
        }
        if (fail) break;
        Item pj = {0, it.t0, it.t0, 0};
        load_item(plan, j, pj);
        sA[n] = pow_f64(dec.lam[h], it.t0 - pj.t1);
        if (fv == 2) {
          sTerm[n++] = -1 - j;
          break;
        }
        sTerm[n++] = j;
      }
    }
    sN = n;
    sFail = fail;
  }
  __syncthreads();  // look-back done (or given up)
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  {
    // the tile as float4s, a fixed set per thread, so every load of a term
    // is in flight at once (d_v tiles are multiples of 4 columns)
    constexpr int NV = NE / 4, PER = (NV + 511) / 512;
    static_assert(DVT % 4 == 0, "float4 rows");
    long long off4[PER];
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int e4 = min(tid + 512 * m, NV - 1);  // a thread past the end repeats the last
      off4[m] = tile_off + (long long)(e4 / (DVT / 4)) * dv + 4 * (e4 % (DVT / 4));
    }
    const bool mine_last = tid + 512 * (PER - 1) < NV;  // its last float4 is its own
    const int nt = sN;
    const bool fail = sFail != 0;
    float4 S[PER];
#pragma unroll
    for (int m = 0; m < PER; ++m) S[m] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int t = 0; t < nt; ++t) {
      const int tm = sTerm[t];
      const float a = sA[t];
      const float *src = tm == kS0Term ? (s0 ? s0 + (long long)it.n * item_stride : nullptr)
                         : tm < 0     ? incl + (long long)(-1 - tm) * item_stride
                                      : slots + (long long)tm * item_stride;
      if (!src) continue;  // no s0: zeros
      float4 x[PER];
#pragma unroll
      for (int m = 0; m < PER; ++m) x[m] = *reinterpret_cast<const float4 *>(src + off4[m]);
#pragma unroll
      for (int m = 0; m < PER; ++m) {
        S[m].x = fmaf(a, x[m].x, S[m].x);
        S[m].y = fmaf(a, x[m].y, S[m].y);
        S[m].z = fmaf(a, x[m].z, S[m].z);
        S[m].w = fmaf(a, x[m].w, S[m].w);
      }
    }
    if (fail) {
      const float nan = __builtin_nanf("");
#pragma unroll
      for (int m = 0; m < PER; ++m) S[m] = make_float4(nan, nan, nan, nan);
    }
    const float aI = pow_f64(dec.lam[h], it.t1 - it.t0);
    float4 Ui[PER];
    if (!last) {
      const float *ui = slots + (long long)idx * item_stride;
#pragma unroll
      for (int m = 0; m < PER; ++m) Ui[m] = *reinterpret_cast<const float4 *>(ui + off4[m]);
    }
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      if (m == PER - 1 && !mine_last) break;
      if (!first)
        *reinterpret_cast<float4 *>(sin + (long long)(idx - 1) * item_stride + off4[m]) = S[m];
      if (!last) {
        float4 y;
        y.x = fmaf(aI, S[m].x, Ui[m].x);
        y.y = fmaf(aI, S[m].y, Ui[m].y);
        y.z = fmaf(aI, S[m].z, Ui[m].z);
        y.w = fmaf(aI, S[m].w, Ui[m].w);
        *reinterpret_cast<float4 *>(incl + (long long)idx * item_stride + off4[m]) = y;
      }
    }
    if (!last) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();  // S_in(i) is written for the output walk's state waves
    if (!last && tid == 0)
      __hip_atomic_store(flag, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // 3. output walk (a sequence's first item reads s0 itself)
  if (role_wave < 4)
    output_role<DVT, false, DKT, GATE>(q, o, gt, gate, it, h, H, dv, c0, scale, tid & 255,
                                       role_wave, sQ, sK, sV, sSt0, sSt1, sPow);
  else
    state_role<DVT, true, false, DKT, KSR>(k, v, s0, s_final, sin, it, idx, h, H, dv, c0,
                                           final_in_slot, tid & 255, role_wave - 4, sK, sKs,
                                           sV, sSt0, sSt1, sPow);
}

template <int DVT, int DKT>
static void launch_chain_dvt(const Plan &p, const FwdArgs &a, const Decay &dec, float *incl,
                             float *sin, int *flags, hipStream_t s) {
  const unsigned grid = (unsigned)((long long)p.max_items * a.H * (a.dv / DVT));
  if (a.gate != kGateNone)
    hipLaunchKernelGGL((fwd_chain_kernel<DVT, DKT, true>), dim3(grid), dim3(512), 0, s,
                       (const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.v, (bf16 *)a.o,
                       a.s0, a.s_final, a.slots, incl, sin, flags, p, dec, a.scale, a.H, a.dv,
                       a.final_in_slot, (const bf16 *)a.g, a.gate);
  else
    hipLaunchKernelGGL((fwd_chain_kernel<DVT, DKT, false>), dim3(grid), dim3(512), 0, s,
                       (const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.v, (bf16 *)a.o,
                       a.s0, a.s_final, a.slots, incl, sin, flags, p, dec, a.scale, a.H, a.dv,
                       a.final_in_slot, (const bf16 *)nullptr, kGateNone);
}

bool fwd_chain_ok(int dk, int H, int items_per_seq) {
  return (dk == 64 || dk == 96) && H % 8 == 0 && items_per_seq <= kChainMaxItems;
}

void launch_fwd_chain(int dvt, const Plan &p, const FwdArgs &a, const Decay &dec, float *incl,
                      float *sin, int *flags, hipStream_t s) {
  if (a.dk == 64) launch_chain_dvt<64, 64>(p, a, dec, incl, sin, flags, s);
  else if (dvt == 96) launch_chain_dvt<96, 96>(p, a, dec, incl, sin, flags, s);
  else launch_chain_dvt<64, 96>(p, a, dec, incl, sin, flags, s);
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
