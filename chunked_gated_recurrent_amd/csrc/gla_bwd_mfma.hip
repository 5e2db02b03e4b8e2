// gla_bwd_mfma.hip -- backward of the chunked Simple GLA forward for bf16
// inputs with dk = 96, 64 or 128 on the gfx950 matrix cores (d_v tiles as
// the forward's: 96 or 64 columns at dk 96, 64 at dk 64 and 128), for the
// heads whose whole d_v does not fit one workgroup of gla_bwd_wide.hip.
//
// The gradients of S_t = lambda S_{t-1} + k_t^T v_t, o_t = scale q_t S_t
// (Laplace 3B / Trainium2 page, sections "GLA mixer" and "Challenge 3":
// training differentiates through every sequential state update) follow
// from G_t = dL/dS_t = lambda G_{t+1} + scale q_t^T dO_t (with dL/dS_final
// entering at the last token):
//     dq_t = scale dO_t S_t^T,   dk_t = v_t G_t^T,   dv_t = k_t G_t,
//     dS0 = lambda G_0.
// Per chunk of L <= 64 tokens (local indices i, t; S_prev the state before
// the chunk, Ch the gradient carried in from the chunks after it):
//     dq_i = scale (lambda^(i+1) dO_i S_prev^T + sum_{j<=i} lambda^(i-j) (dO_i . v_j) k_j)
//     dv_i = lambda^(L-1-i) k_i Ch + scale sum_{t>=i} lambda^(t-i) (q_t . k_i) dO_t
//     dk_i = lambda^(L-1-i) Ch v_i^T + scale sum_{t>=i} lambda^(t-i) (dO_t . v_i) q_t
//     Ch  <- lambda^L Ch + scale sum_t lambda^(t+1) q_t^T dO_t      (for the chunk before)
//
// Two passes, each a workgroup per (sequence, head, dv tile):
//   * bwd_dq_kernel walks the chunks forward: the state role of the forward
//     kernel rebuilds S tile by tile, and four "dq waves" form the dq terms
//     of their 16 rows over this dv tile;
//   * bwd_dkdv_kernel walks the chunks backward with the carried gradient Ch
//     of its dv tile in MFMA accumulators: four "dv waves" form dv (complete:
//     its contraction runs over dk) and advance Ch, four "dk waves" form the
//     dk terms of this dv tile.
// dq and dk contract over dv, so each dv tile yields a partial sum: fp32 rows
// [dv tile][H][token][dk] in the workspace (each lane stores the 4
// consecutive dk values of one token that it holds), which a streaming
// kernel adds up into bf16 dq and dk. (dv = 192 takes the workgroup-per-head
// kernels of gla_bwd_wide.hip instead; this file also holds the boundary
// pass that gives time segments their incoming states and carries, used by
// both.)
#include "gla_mfma.h"

namespace gla {

// fp32 partial-sum rows: [dv tile][H][total tokens][dk]
__device__ __forceinline__ float *part_row(float *part, int dtile, int h, long long t,
                                           int H, long long total_T, int dk) {
  return part + (((long long)dtile * H + h) * total_T + t) * dk;
}

// ---------------------------------------------------------------------------
// dq role: 4 waves (role wave w owns rows 16 w .. 16 w + 15 of a chunk).
// ---------------------------------------------------------------------------
template <int DVT, int DKT>
__device__ __forceinline__ void dq_role(
    const bf16 *__restrict__ dout, float *__restrict__ part, const Item &it,
    int h, int H, int dv, int c0, int dtile, long long total_T, float scale,
    int rt, int w, bf16 *sD,
    const bf16 *sK, const bf16 *sV, const bf16 *sSt0, const bf16 *sSt1,
    const float *sPow) {
  using M = MfCfg<DVT, DKT>;
  constexpr int C = M::C, QS = M::QS, VS = M::VS;
  constexpr int NDT = M::NDT, NJS = M::NJS, NVV = M::NVV, VV = M::VV;
  constexpr int NCS = DVT / 32;  // 32-deep steps over the dv tile
  const int lane = rt & 63, l16 = lane & 15, g = lane >> 4;
  const int tr_row = l16 >> 2, tr_col = 4 * (l16 & 3);
  const unsigned rowVb = (unsigned)(H * dv * 2);
  const int nch = (it.t1 - it.t0 + C - 1) / C;

  int rowD[VV], colD[VV];
#pragma unroll
  for (int m = 0; m < VV; ++m) {
    const int vi = rt + 256 * m;
    rowD[m] = vi / NVV;
    colD[m] = vi - rowD[m] * NVV;
  }
  auto load_d = [&](int ch, u32x4(&r)[VV]) {
    const long long tb = (long long)it.t0 + (long long)ch * C;
    const __amdgpu_buffer_rsrc_t bd =
        buf_rsrc(dout + tb * H * dv + (long long)h * dv + c0,
                 (unsigned)chunk_rows(it, ch) * rowVb);
#pragma unroll
    for (int m = 0; m < VV; ++m)
      r[m] = __builtin_amdgcn_raw_buffer_load_b128(bd, rowD[m] * rowVb + colD[m] * 16, 0, 0);
  };
  constexpr int KBUF = C * QS, VBUF = C * VS;
  auto store_d = [&](int buf, const u32x4(&r)[VV]) {
#pragma unroll
    for (int m = 0; m < VV; ++m)
      *reinterpret_cast<u32x4 *>(sD + buf * VBUF + rowD[m] * VS + 8 * colD[m]) = r[m];
  };

  u32x4 ra[VV], rb[VV];
  load_d(0, ra);
  load_d(1, rb);
  __syncthreads();  // sPow ready
  const int i_row = 16 * w + l16;
  const float lam_i1 = sPow[i_row + 1];
  float maskw[4][4];  // lambda^(i-j) for j <= i, else 0 (this lane's column i)
#pragma unroll
  for (int J = 0; J < 4; ++J)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int diff = i_row - (16 * J + 4 * g + r);
      maskw[J][r] = diff >= 0 ? sPow[max(diff, 0)] : 0.f;
    }
  store_d(0, ra);

  auto body = [&](int ch, u32x4(&rnew)[VV], const u32x4(&rnext)[VV], const bf16 *st) {
    const int cur = ch & 1;
    __syncthreads();  // chunk ch and S_{ch-1} are in LDS; chunk ch-1 is done
    load_d(ch + 2, rnew);
    store_d(cur ^ 1, rnext);
    const bf16 *cD = sD + cur * VBUF, *cK = sK + cur * KBUF, *cV = sV + cur * VBUF;
    // dO row i over this dv tile: natural k-set (scores) and P k-set (S term)
    bf16x8 dfn[NCS], dfp[NCS];
#pragma unroll
    for (int s = 0; s < NCS; ++s) {
      const int row = i_row * VS + 32 * s;
      dfn[s] = *reinterpret_cast<const bf16x8 *>(cD + row + 8 * g);
      dfp[s] = cat8(lds8_apart(cD, row + 4 * g), lds8_apart(cD, row + 16 + 4 * g));
    }
    // P'^T[j][i] = v_j . dO_i over the tile, for j blocks 0..3
    f32x4 p[4];
#pragma unroll
    for (int J = 0; J < 4; ++J) p[J] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NCS; ++s)
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        const bf16x8 vfr = *reinterpret_cast<const bf16x8 *>(cV + (16 * J + l16) * VS + 32 * s + 8 * g);
        p[J] = mfma(vfr, dfn[s], p[J]);
      }
    bf16x8 pb[NJS];
#pragma unroll
    for (int s = 0; s < NJS; ++s)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pb[s][r] = (bf16)(p[2 * s][r] * maskw[2 * s][r]);
        pb[s][4 + r] = (bf16)(p[2 * s + 1][r] * maskw[2 * s + 1][r]);
      }
    // dq^T[d][i] = lambda^(i+1) (S dO^T)[d][i] + (K^T P'^T)[d][i]
    f32x4 acc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NCS; ++s)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const bf16 *base = st + (32 * s + 4 * g + tr_row) * QS + 16 * dt + tr_col;
        acc[dt] = mfma(cat8(tr4(base), tr4(base + 16 * QS)), dfp[s], acc[dt]);
      }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[dt] *= lam_i1;
#pragma unroll
    for (int s = 0; s < NJS; ++s)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const bf16 *base = cK + (32 * s + 4 * g + tr_row) * QS + 16 * dt + tr_col;
        acc[dt] = mfma(cat8(tr4(base), tr4(base + 16 * QS)), pb[s], acc[dt]);
      }
    // partial dq of this dv tile: this lane holds dk values 16 dt + 4 g .. +3
    // of token i_row (rows past the item's end are not written: they belong
    // to the next item or sequence)
    if (i_row < chunk_rows(it, ch)) {
      float *dst = part_row(part, dtile, h, it.t0 + (long long)ch * C + i_row, H, total_T, M::DK) + 4 * g;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        *reinterpret_cast<f32x4 *>(dst + 16 * dt) = acc[dt] * scale;
    }
  };
  for (int ch = 0; ch < nch; ch += 2) {  // a past-the-end chunk is all zeros
    body(ch, ra, rb, sSt1);               // reads S_{ch-1}
    body(ch + 1, rb, ra, sSt0);
  }
}

template <int DVT, int DKT>
__global__ __launch_bounds__(512, 1) void bwd_dq_kernel(
    const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const bf16 *__restrict__ dout, const float *__restrict__ s0,
    float *__restrict__ slots, float *__restrict__ part_dq, Plan plan,
    Decay dec, float scale, int H, int dv) {
  using M = MfCfg<DVT, DKT>;
  __shared__ __attribute__((aligned(16))) bf16 sD[2 * M::C * M::VS];
  __shared__ __attribute__((aligned(16))) bf16 sK[2 * M::C * M::QS];
  __shared__ __attribute__((aligned(16))) bf16 sKs[2 * M::C * M::QS];
  __shared__ __attribute__((aligned(16))) bf16 sV[2 * M::C * M::VS];
  __shared__ __attribute__((aligned(16))) bf16 sSt0[DVT * M::QS];
  __shared__ __attribute__((aligned(16))) bf16 sSt1[DVT * M::QS];
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
    dq_role<DVT, DKT>(dout, part_dq, it, h, H, dv, c0, dtile, plan.total_T, scale, tid & 255,
                 role_wave, sD, sK, sV, sSt0, sSt1, sPow);
  else
    state_role<DVT, true, false, DKT>(k, v, s0, nullptr, slots, it, idx, h, H, dv, c0, 0,
                          tid & 255, role_wave - 4, sK, sKs, sV, sSt0, sSt1, sPow);
}

// ---------------------------------------------------------------------------
// Reverse walk: dv waves (dv of 16 rows + the carried gradient Ch) and dk
// waves (partial dk of 16 rows), chunks from the last to the first.
// ---------------------------------------------------------------------------
template <int DVT, int DKT>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k,
    const bf16 *__restrict__ v, const bf16 *__restrict__ dout,
    const float *__restrict__ ds_final, const float *__restrict__ cslots,
    bf16 *__restrict__ dv_out, float *__restrict__ ds0,
    float *__restrict__ part_dk, Plan plan, Decay dec, float scale, int H,
    int dv) {
  using M = MfCfg<DVT, DKT>;
  constexpr int C = M::C, DK = M::DK, QS = M::QS, VS = M::VS;
  constexpr int NDT = M::NDT, NCT = M::NCT, NJS = M::NJS, NKS = M::NKS;
  constexpr int SDT = M::SDT, SCT = M::SCT, QV = M::QV, VV = M::VV, NVV = M::NVV;
  constexpr int NCS = DVT / 32;
  constexpr int KBUF = C * QS, VBUF = C * VS;
  __shared__ __attribute__((aligned(16))) bf16 sQ[2 * C * QS];
  __shared__ __attribute__((aligned(16))) bf16 sK[2 * C * QS];
  __shared__ __attribute__((aligned(16))) bf16 sV[2 * C * VS];
  __shared__ __attribute__((aligned(16))) bf16 sD[2 * C * VS];
  __shared__ __attribute__((aligned(16))) bf16 sCt0[DVT * QS];
  __shared__ __attribute__((aligned(16))) bf16 sCt1[DVT * QS];
  __shared__ float sPow[C + 4];

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
  if (tid <= C) sPow[tid] = pow_f64(dec.lam[h], tid);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool dv_role = wave < 4;
  const int w = wave & 3, rt = tid & 255;
  const int lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int tr_row = l16 >> 2, tr_col = 4 * (l16 & 3);
  const int c0 = dtile * DVT;
  const unsigned rowKb = (unsigned)(H * DK * 2), rowVb = (unsigned)(H * dv * 2);
  const int nch = (it.t1 - it.t0 + C - 1) / C;
  const int i_row = 16 * w + l16;
  const long long state_off = ((long long)it.n * H + h) * DK * dv;

  // Chunk rows; chunks before the first (ch < 0) are empty.
  auto rows_of = [&](int ch) { return ch < 0 ? 0 : chunk_rows(it, ch); };

  // loads: dv waves bring q and k, dk waves v and dO
  int rowA[QV], colA[QV], rowB[VV], colB[VV];
#pragma unroll
  for (int m = 0; m < QV; ++m) {
    const int vi = rt + 256 * m;
    rowA[m] = vi / M::NQV;
    colA[m] = vi - rowA[m] * M::NQV;
  }
#pragma unroll
  for (int m = 0; m < VV; ++m) {
    const int vi = rt + 256 * m;
    rowB[m] = vi / NVV;
    colB[m] = vi - rowB[m] * NVV;
  }
  // Per-lane byte offsets of the role's 16-byte loads. Both roles issue the
  // same QV loads per operand into the same stage registers (a role-dependent
  // count makes the compiler keep the stage arrays in private memory); the
  // slots the dk role does not need (d_v tiles narrower than d_k) point past
  // every buffer's end, where a buffer load returns zeros and reads nothing.
  static_assert(VV <= QV, "a d_v tile is at most d_k wide");
  unsigned offs[QV];
#pragma unroll
  for (int m = 0; m < QV; ++m) {
    unsigned ob = 0x80000000u;
    if (m < VV) ob = rowB[m < VV ? m : 0] * rowVb + colB[m < VV ? m : 0] * 16;
    offs[m] = dv_role ? rowA[m] * rowKb + colA[m] * 16 : ob;
  }
  auto load = [&](int ch, u32x4(&r1)[QV], u32x4(&r2)[QV]) {
    const int L = rows_of(ch);
    const long long tb = (long long)it.t0 + (long long)(ch < 0 ? 0 : ch) * C;
    const long long vo = tb * H * dv + (long long)h * dv + c0;
    const long long ko = (tb * H + h) * DK;
    const __amdgpu_buffer_rsrc_t b1 =
        buf_rsrc(dv_role ? q + ko : v + vo, (unsigned)L * (dv_role ? rowKb : rowVb));
    const __amdgpu_buffer_rsrc_t b2 =
        buf_rsrc(dv_role ? k + ko : dout + vo, (unsigned)L * (dv_role ? rowKb : rowVb));
#pragma unroll
    for (int m = 0; m < QV; ++m) r1[m] = __builtin_amdgcn_raw_buffer_load_b128(b1, offs[m], 0, 0);
#pragma unroll
    for (int m = 0; m < QV; ++m) r2[m] = __builtin_amdgcn_raw_buffer_load_b128(b2, offs[m], 0, 0);
  };
  auto store = [&](int buf, const u32x4(&r1)[QV], const u32x4(&r2)[QV]) {
    if (dv_role) {
#pragma unroll
      for (int m = 0; m < QV; ++m) {
        *reinterpret_cast<u32x4 *>(sQ + buf * KBUF + rowA[m] * QS + 8 * colA[m]) = r1[m];
        *reinterpret_cast<u32x4 *>(sK + buf * KBUF + rowA[m] * QS + 8 * colA[m]) = r2[m];
      }
    } else {
#pragma unroll
      for (int m = 0; m < VV; ++m) {
        *reinterpret_cast<u32x4 *>(sV + buf * VBUF + rowB[m] * VS + 8 * colB[m]) = r1[m];
        *reinterpret_cast<u32x4 *>(sD + buf * VBUF + rowB[m] * VS + 8 * colB[m]) = r2[m];
      }
    }
  };

  // carried gradient Ch (dv waves): SDT x SCT tiles of 16 x 16, fp32. It
  // starts as dL/dS_final for a sequence's last item, else as the combined
  // carry flowing out of the next item (its slot)
  const int dt0 = SDT * (w >> 1), ct0 = SCT * (w & 1);
  const float *cin = (it.flags & kLastSeg)
                         ? (ds_final ? ds_final + state_off : nullptr)
                         : cslots + ((long long)(idx + 1) * H + h) * DK * dv;
  f32x4 accC[SDT][SCT];
#pragma unroll
  for (int a = 0; a < SDT; ++a)
#pragma unroll
    for (int b = 0; b < SCT; ++b) {
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
      if (dv_role && cin) {
        const int d = 16 * (dt0 + a) + 4 * g;
        const int c = c0 + 16 * (ct0 + b) + l16;
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = cin[(long long)(d + r) * dv + c];
      }
      accC[a][b] = x;
    }
  auto publish = [&](bf16 *dst) {  // Ch^T as bf16, row c, columns d
#pragma unroll
    for (int a = 0; a < SDT; ++a)
#pragma unroll
      for (int b = 0; b < SCT; ++b) {
        bf16x4 t;
#pragma unroll
        for (int r = 0; r < 4; ++r) t[r] = (bf16)accC[a][b][r];
        const int c = 16 * (ct0 + b) + l16;
        *reinterpret_cast<bf16x4 *>(dst + c * QS + 16 * (dt0 + a) + 4 * g) = t;
      }
  };

  u32x4 a1[QV], a2[QV], b1[QV], b2[QV];
  load(nch - 1, a1, a2);
  load(nch - 2, b1, b2);
  __syncthreads();  // sPow ready
  // scores mask: scale * lambda^(t-i) for t >= i, else 0 (column i of this lane)
  float maskA[4][4];
#pragma unroll
  for (int T = 0; T < 4; ++T)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int diff = (16 * T + 4 * g + r) - i_row;
      maskA[T][r] = diff >= 0 ? scale * sPow[max(diff, 0)] : 0.f;
    }
  // carry scaling of q_t: scale * lambda^(t+1) for this lane's P k-set rows t
  float fq[NJS][8];
#pragma unroll
  for (int s = 0; s < NJS; ++s)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      fq[s][e] = scale * sPow[32 * s + 4 * g + e + 1];
      fq[s][4 + e] = scale * sPow[32 * s + 16 + 4 * g + e + 1];
    }
  store((nch - 1) & 1, a1, a2);
  if (dv_role) publish(sCt0);

  // step p processes chunk ch = nch - 1 - p: reads Ch from sCt[p & 1] and
  // publishes the advanced Ch into sCt[(p + 1) & 1]
  auto body = [&](int ch, u32x4(&n1)[QV], u32x4(&n2)[QV], const u32x4(&x1)[QV],
                  const u32x4(&x2)[QV], const bf16 *ct_in, bf16 *ct_out) {
    const int L = rows_of(ch);
    const int cur = ch & 1;
    const long long tb = (long long)it.t0 + (long long)(ch < 0 ? 0 : ch) * C;
    __syncthreads();  // chunk ch and Ch_in are in LDS; the chunk after is done
    load(ch - 2, n1, n2);
    store(cur ^ 1, x1, x2);
    const bf16 *cQ = sQ + cur * KBUF, *cK = sK + cur * KBUF;
    const bf16 *cV = sV + cur * VBUF, *cD = sD + cur * VBUF;
    const float lam_rev = sPow[clampi(L - 1 - i_row, 0, C)];  // lambda^(L-1-i)
    if (dv_role) {
      // scores A[t][i] = q_t . k_i (natural k-set over d)
      bf16x8 kf[NKS];
#pragma unroll
      for (int s = 0; s < NKS; ++s)
        kf[s] = *reinterpret_cast<const bf16x8 *>(cK + i_row * QS + 32 * s + 8 * g);
      f32x4 sc[4];
#pragma unroll
      for (int T = 0; T < 4; ++T) sc[T] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NKS; ++s)
#pragma unroll
        for (int T = 0; T < 4; ++T) {
          const bf16x8 qf = *reinterpret_cast<const bf16x8 *>(cQ + (16 * T + l16) * QS + 32 * s + 8 * g);
          sc[T] = mfma(qf, kf[s], sc[T]);
        }
      bf16x8 ab[NJS];
#pragma unroll
      for (int s = 0; s < NJS; ++s)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          ab[s][r] = (bf16)(sc[2 * s][r] * maskA[2 * s][r]);
          ab[s][4 + r] = (bf16)(sc[2 * s + 1][r] * maskA[2 * s + 1][r]);
        }
      // dv^T[c][i] = lambda^(L-1-i) (Ch^T K^T)[c][i] + (dO^T A)[c][i]
      f32x4 acc[NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) acc[ct] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NKS; ++s)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const bf16x8 cf = *reinterpret_cast<const bf16x8 *>(ct_in + (16 * ct + l16) * QS + 32 * s + 8 * g);
          acc[ct] = mfma(cf, kf[s], acc[ct]);
        }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) acc[ct] *= lam_rev;
#pragma unroll
      for (int s = 0; s < NJS; ++s)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const bf16 *base = cD + (32 * s + 4 * g + tr_row) * VS + 16 * ct + tr_col;
          acc[ct] = mfma(cat8(tr4(base), tr4(base + 16 * VS)), ab[s], acc[ct]);
        }
      // Ch <- lambda^L Ch + scale sum_t lambda^(t+1) q_t^T dO_t
      const float lamL = sPow[L];
#pragma unroll
      for (int a = 0; a < SDT; ++a)
#pragma unroll
        for (int b = 0; b < SCT; ++b) accC[a][b] *= lamL;
#pragma unroll
      for (int s = 0; s < NJS; ++s) {
        bf16x8 qa[SDT], dfr[SCT];
        const int row = 32 * s + 4 * g + tr_row;
#pragma unroll
        for (int a = 0; a < SDT; ++a) {
          const bf16 *base = cQ + row * QS + 16 * (dt0 + a) + tr_col;
          const bf16x8 raw = cat8(tr4(base), tr4(base + 16 * QS));
#pragma unroll
          for (int e = 0; e < 8; ++e) qa[a][e] = (bf16)((float)raw[e] * fq[s][e]);
        }
#pragma unroll
        for (int b = 0; b < SCT; ++b) {
          const bf16 *base = cD + row * VS + 16 * (ct0 + b) + tr_col;
          dfr[b] = cat8(tr4(base), tr4(base + 16 * VS));
        }
#pragma unroll
        for (int a = 0; a < SDT; ++a)
#pragma unroll
          for (int b = 0; b < SCT; ++b) accC[a][b] = mfma(qa[a], dfr[b], accC[a][b]);
      }
      publish(ct_out);
      // stage dv rows of this wave in its own rows of the k tile (only this
      // wave reads them, and kf is loaded), then 16-byte row segments
      bf16 *so = const_cast<bf16 *>(cK) + 16 * w * QS;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        bf16x4 t;
#pragma unroll
        for (int r = 0; r < 4; ++r) t[r] = (bf16)acc[ct][r];
        *reinterpret_cast<bf16x4 *>(so + l16 * QS + 16 * ct + 4 * g) = t;
      }
      const __amdgpu_buffer_rsrc_t bo =
          buf_rsrc(dv_out + tb * H * dv + (long long)h * dv + c0, (unsigned)L * rowVb);
#pragma unroll
      for (int m = 0; m < M::OV; ++m) {
        const int vi = lane + 64 * m;
        const int row = vi / NVV, col = vi - (vi / NVV) * NVV;
        const u32x4 val = *reinterpret_cast<const u32x4 *>(so + row * QS + 8 * col);
        __builtin_amdgcn_raw_buffer_store_b128(val, bo, (16 * w + row) * rowVb + col * 16, 0, 0);
      }
    } else {
      // scores Bm[t][i] = dO_t . v_i over this dv tile (natural k-set over
      // c: both operands are 16-byte row reads)
      f32x4 sc[4];
#pragma unroll
      for (int T = 0; T < 4; ++T) sc[T] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NCS; ++s) {
        const bf16x8 vn = *reinterpret_cast<const bf16x8 *>(cV + i_row * VS + 32 * s + 8 * g);
#pragma unroll
        for (int T = 0; T < 4; ++T) {
          const bf16x8 df =
              *reinterpret_cast<const bf16x8 *>(cD + (16 * T + l16) * VS + 32 * s + 8 * g);
          sc[T] = mfma(df, vn, sc[T]);
        }
      }
      bf16x8 bm[NJS];
#pragma unroll
      for (int s = 0; s < NJS; ++s)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          bm[s][r] = (bf16)(sc[2 * s][r] * maskA[2 * s][r]);
          bm[s][4 + r] = (bf16)(sc[2 * s + 1][r] * maskA[2 * s + 1][r]);
        }
      // dk^T[d][i] = lambda^(L-1-i) (Ch V^T)[d][i] + (Q^T Bm)[d][i]
      f32x4 acc[NDT];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) acc[dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NCS; ++s) {
        // v_i in the P k-set over c, matching the transposed reads of Ch
        const int vrow = i_row * VS + 32 * s;
        const bf16x8 vf = cat8(lds8_apart(cV, vrow + 4 * g), lds8_apart(cV, vrow + 16 + 4 * g));
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const bf16 *base = ct_in + (32 * s + 4 * g + tr_row) * QS + 16 * dt + tr_col;
          acc[dt] = mfma(cat8(tr4(base), tr4(base + 16 * QS)), vf, acc[dt]);
        }
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) acc[dt] *= lam_rev;
#pragma unroll
      for (int s = 0; s < NJS; ++s)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const bf16 *base = cQ + (32 * s + 4 * g + tr_row) * QS + 16 * dt + tr_col;
          acc[dt] = mfma(cat8(tr4(base), tr4(base + 16 * QS)), bm[s], acc[dt]);
        }
      if (i_row < L) {  // rows past the item's end are not written
        float *dst = part_row(part_dk, dtile, h, tb + i_row, H, plan.total_T, M::DK) + 4 * g;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) *reinterpret_cast<f32x4 *>(dst + 16 * dt) = acc[dt];
      }
    }
  };
  for (int p = 0; p < nch; p += 2) {  // a chunk before the first is all zeros
    body(nch - 1 - p, a1, a2, b1, b2, sCt0, sCt1);
    body(nch - 2 - p, b1, b2, a1, a2, sCt1, sCt0);
  }
  // after the first chunk Ch is dL/dS0 (an extra empty step leaves it as is:
  // lambda^0 = 1 and no rows)
  if (dv_role && ds0 && (it.flags & kFirstSeg)) {
#pragma unroll
    for (int a = 0; a < SDT; ++a)
#pragma unroll
      for (int b = 0; b < SCT; ++b) {
        const int d = 16 * (dt0 + a) + 4 * g;
        const int c = c0 + 16 * (ct0 + b) + l16;
#pragma unroll
        for (int r = 0; r < 4; ++r) ds0[state_off + (long long)(d + r) * dv + c] = accC[a][b][r];
      }
  }
}

// ---------------------------------------------------------------------------
// Local carries of time segments: for every item but a sequence's first,
// U_g = scale sum_{t in item} lambda^(t - t0 + 1) q_t^T dO_t (the carried
// gradient the item passes back when nothing flows into it), into slot g.
// A plain weighted sum, so the chunks are taken first to last (chunk c
// weighted by lambda^(64 c) on top of its in-chunk powers): the walk ends on
// the item's last rows, where the reverse walk that consumes the carry starts
// next, so those rows are still in the last-level cache.
// ---------------------------------------------------------------------------
template <int DVT, int DKT>
__device__ __forceinline__ void carry_role(
    const bf16 *__restrict__ q, const bf16 *__restrict__ dout, float *__restrict__ cslots,
    const Item &it, int idx, int h, int dtile, float scale, int H, int dv, int tid,
    bf16 *sQ, bf16 *sD, const float *sPow) {
  using M = MfCfg<DVT, DKT>;
  constexpr int C = M::C, DK = M::DK, QS = M::QS, VS = M::VS;
  constexpr int NJS = M::NJS, SDT = M::SDT, SCT = M::SCT, QV = M::QV, VV = M::VV;
  constexpr int NVV = M::NVV;
  constexpr int KBUF = C * QS, VBUF = C * VS;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int tr_row = l16 >> 2, tr_col = 4 * (l16 & 3);
  const int c0 = dtile * DVT;
  const unsigned rowKb = (unsigned)(H * DK * 2), rowVb = (unsigned)(H * dv * 2);
  const int nch = (it.t1 - it.t0 + C - 1) / C;
  const int dt0 = SDT * (w >> 1), ct0 = SCT * (w & 1);
  auto rows_of = [&](int ch) { return ch < 0 ? 0 : chunk_rows(it, ch); };

  int rowA[QV], colA[QV], rowB[VV], colB[VV];
#pragma unroll
  for (int m = 0; m < QV; ++m) {
    const int vi = tid + 256 * m;
    rowA[m] = vi / M::NQV;
    colA[m] = vi - rowA[m] * M::NQV;
  }
#pragma unroll
  for (int m = 0; m < VV; ++m) {
    const int vi = tid + 256 * m;
    rowB[m] = vi / NVV;
    colB[m] = vi - rowB[m] * NVV;
  }
  auto load = [&](int ch, u32x4(&rq)[QV], u32x4(&rd)[VV]) {
    const unsigned L = (unsigned)rows_of(ch);
    const long long tb = (long long)it.t0 + (long long)(ch < 0 ? 0 : ch) * C;
    const __amdgpu_buffer_rsrc_t bq = buf_rsrc(q + (tb * H + h) * DK, L * rowKb);
    const __amdgpu_buffer_rsrc_t bd =
        buf_rsrc(dout + tb * H * dv + (long long)h * dv + c0, L * rowVb);
#pragma unroll
    for (int m = 0; m < QV; ++m)
      rq[m] = __builtin_amdgcn_raw_buffer_load_b128(bq, rowA[m] * rowKb + colA[m] * 16, 0, 0);
#pragma unroll
    for (int m = 0; m < VV; ++m)
      rd[m] = __builtin_amdgcn_raw_buffer_load_b128(bd, rowB[m] * rowVb + colB[m] * 16, 0, 0);
  };
  // q enters the carry only as scale * lambda^(t - t0 + 1) q_t: it is stored
  // scaled, by its in-chunk power times the chunk's lambda^(64 c) (pc)
  float fqr[QV];
  auto store = [&](int buf, float pc, const u32x4(&rq)[QV], const u32x4(&rd)[VV]) {
#pragma unroll
    for (int m = 0; m < QV; ++m) {
      const bf16x8 qv = __builtin_bit_cast(bf16x8, rq[m]);
      const float f = fqr[m] * pc;
      bf16x8 qs;
#pragma unroll
      for (int e = 0; e < 8; ++e) qs[e] = (bf16)((float)qv[e] * f);
      *reinterpret_cast<bf16x8 *>(sQ + buf * KBUF + rowA[m] * QS + 8 * colA[m]) = qs;
    }
#pragma unroll
    for (int m = 0; m < VV; ++m)
      *reinterpret_cast<u32x4 *>(sD + buf * VBUF + rowB[m] * VS + 8 * colB[m]) = rd[m];
  };

  f32x4 accC[SDT][SCT];
#pragma unroll
  for (int a = 0; a < SDT; ++a)
#pragma unroll
    for (int b = 0; b < SCT; ++b) accC[a][b] = (f32x4){0.f, 0.f, 0.f, 0.f};
  u32x4 qa_[QV], da_[VV], qb_[QV], db_[VV];
  load(0, qa_, da_);
  load(1, qb_, db_);
  __syncthreads();  // sPow ready
#pragma unroll
  for (int m = 0; m < QV; ++m) fqr[m] = scale * sPow[rowA[m] + 1];
  // lambda^(64 c) for the chunk whose rows are stored next (underflows to
  // zero harmlessly for strong decay)
  const float lam64 = sPow[C];
  float pc = 1.0f;
  store(0, pc, qa_, da_);

  auto body = [&](int ch, u32x4(&nq)[QV], u32x4(&nd)[VV], const u32x4(&xq)[QV],
                  const u32x4(&xd)[VV]) {
    const int cur = ch & 1;
    __syncthreads();  // chunk ch is in LDS; the chunk before is done
    load(ch + 2, nq, nd);
    pc *= lam64;
    store(cur ^ 1, pc, xq, xd);
    const bf16 *cQ = sQ + cur * KBUF, *cD = sD + cur * VBUF;
#pragma unroll
    for (int s = 0; s < NJS; ++s) {
      bf16x8 qs[SDT], dfr[SCT];
      const int row = 32 * s + 4 * g + tr_row;
#pragma unroll
      for (int a = 0; a < SDT; ++a) {
        const bf16 *base = cQ + row * QS + 16 * (dt0 + a) + tr_col;
        qs[a] = cat8(tr4(base), tr4(base + 16 * QS));
      }
#pragma unroll
      for (int b = 0; b < SCT; ++b) {
        const bf16 *base = cD + row * VS + 16 * (ct0 + b) + tr_col;
        dfr[b] = cat8(tr4(base), tr4(base + 16 * VS));
      }
#pragma unroll
      for (int a = 0; a < SDT; ++a)
#pragma unroll
        for (int b = 0; b < SCT; ++b) accC[a][b] = mfma(qs[a], dfr[b], accC[a][b]);
    }
  };
  for (int ch = 0; ch < nch; ch += 2) {  // a chunk past the end is all zeros
    body(ch, qa_, da_, qb_, db_);
    body(ch + 1, qb_, db_, qa_, da_);
  }
  float *dst = cslots + ((long long)idx * H + h) * DK * dv;
#pragma unroll
  for (int a = 0; a < SDT; ++a)
#pragma unroll
    for (int b = 0; b < SCT; ++b) {
      const int d = 16 * (dt0 + a) + 4 * g;
      const int c = c0 + 16 * (ct0 + b) + l16;
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[(long long)(d + r) * dv + c] = accC[a][b][r];
    }
}

// ---------------------------------------------------------------------------
// Time segments, both directions in one launch: workgroups [0, n_state) run
// the forward's state pass (local end state of every segment but a
// sequence's last, into `slots`), the rest the local carries (every segment
// but a sequence's first, into `cslots`). The two halves read different
// arrays (k, v and q, dO) and each leaves half of the unit slots idle, so
// together they fill the GPU once instead of half-filling it twice.
// ---------------------------------------------------------------------------
template <int DVT, int DKT>
__global__ __launch_bounds__(256, 2) void bwd_boundary_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const bf16 *__restrict__ dout, float *__restrict__ slots, float *__restrict__ cslots,
    Plan plan, Decay dec, float scale, int H, int dv, int n_state) {
  using M = MfCfg<DVT, DKT>;
  __shared__ __attribute__((aligned(16))) bf16 sA[2 * M::C * M::QS];
  __shared__ __attribute__((aligned(16))) bf16 sB[2 * M::C * M::VS];
  __shared__ float sPow[M::C + 4];
  const bool state = (int)blockIdx.x < n_state;
  const int P = state ? (int)blockIdx.x : (int)blockIdx.x - n_state;
  const int ndt = dv / DVT;
  int unit, dtile;
  xcd_unit_at(plan, P, ndt, plan.max_items * H, unit, dtile);
  if (unit >= plan.max_items * H) return;
  const int slot = unit / H;
  const int h = unit - slot * H;
  int idx;
  Item it;
  if (!slot_item(plan, slot, idx, it)) return;
  make_uniform(idx, it);
  // no later segment reads a last segment's state, no earlier one a first
  // segment's carry
  if (it.flags & (state ? kLastSeg : kFirstSeg)) return;
  const int tid = threadIdx.x;
  if (tid <= M::C) sPow[tid] = pow_f64(dec.lam[h], tid);
  if (state)
    state_role<DVT, false, false, DKT>(k, v, nullptr, nullptr, slots, it, idx, h, H, dv, dtile * DVT, 0,
                           tid, __builtin_amdgcn_readfirstlane(tid >> 6), nullptr, sA, sB,
                           nullptr, nullptr, sPow);
  else
    carry_role<DVT, DKT>(q, dout, cslots, it, idx, h, dtile, scale, H, dv, tid, sA, sB, sPow);
}

// ---------------------------------------------------------------------------
// dq, dk <- sum of the dv-tile partials, as bf16 in [tokens, H, dk]
// ---------------------------------------------------------------------------
// One thread per 4 consecutive values of one (token, head) row; each partial
// is read once (non-temporal loads).
__global__ __launch_bounds__(256) void bwd_reduce_kernel(
    const float *__restrict__ part_dq, const float *__restrict__ part_dk,
    bf16 *__restrict__ dq, bf16 *__restrict__ dk, long long total_T, int H, int ndt,
    int dkd) {
  typedef float f32x4n __attribute__((ext_vector_type(4)));
  const int q4 = dkd / 4;  // float4s per (token, head) row
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;  // float4 index
  const long long n4 = total_T * H * q4;
  if (e >= n4) return;
  const long long row = e / q4;  // token * H + head
  const int c4 = (int)(e - row * q4);
  const long long t = row / H;
  const int h = (int)(row - t * H);
  f32x4n sq = {0.f, 0.f, 0.f, 0.f}, sk = {0.f, 0.f, 0.f, 0.f};
  for (int d = 0; d < ndt; ++d) {
    const long long off = (((long long)d * H + h) * total_T + t) * dkd + 4 * c4;
    sq += __builtin_nontemporal_load(reinterpret_cast<const f32x4n *>(part_dq + off));
    sk += __builtin_nontemporal_load(reinterpret_cast<const f32x4n *>(part_dk + off));
  }
  bf16x4 oq, ok;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    oq[r] = (bf16)sq[r];
    ok[r] = (bf16)sk[r];
  }
  *reinterpret_cast<bf16x4 *>(dq + row * dkd + 4 * c4) = oq;
  *reinterpret_cast<bf16x4 *>(dk + row * dkd + 4 * c4) = ok;
}

template <int DVT, int DKT>
static void launch_boundary_dvt(const Plan &p, const BwdArgs &a, const Decay &dec,
                                hipStream_t s) {
  Plan pb = p;
  pb.deal = 1;  // both halves skip a segment of every sequence
  const unsigned g = xcd_grid(1, (long long)p.max_items * a.H, a.dv / DVT);
  hipLaunchKernelGGL((bwd_boundary_kernel<DVT, DKT>), dim3(2 * g), dim3(256), 0, s,
                     (const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.v,
                     (const bf16 *)a.dout, a.slots, a.cslots, pb, dec, a.scale, a.H, a.dv,
                     (int)g);
}

// d_v tiles as the forward's (96 or 64 columns at dk 96, 64 at dk 64 and
// 128), except dk 96 with dv 128 (always the per-head backward): one tile
// of all 128 columns, so q and k are requested once per token instead of
// once per tile (66 KB of LDS, two workgroups per CU). The same at dv 192
// (82 KB, one workgroup per CU) measured slower than two 96-column tiles.
hipError_t launch_bwd_boundary(int dvt, const Plan &p, const BwdArgs &a, const Decay &dec,
                               hipStream_t s) {
  if (a.dk_dim == 96 && a.dv == 128) launch_boundary_dvt<128, 96>(p, a, dec, s);
  else if (a.dk_dim == 64) launch_boundary_dvt<64, 64>(p, a, dec, s);
  else if (a.dk_dim == 128) launch_boundary_dvt<64, 128>(p, a, dec, s);
  else if (dvt == 96) launch_boundary_dvt<96, 96>(p, a, dec, s);
  else launch_boundary_dvt<64, 96>(p, a, dec, s);
  return hipGetLastError();
}

template <int DVT, int DKT>
static void launch_bwd_dvt(const Plan &p, const BwdArgs &a, const Decay &dec,
                           hipStream_t s) {
  const unsigned grid = xcd_grid(p.deal, (long long)p.max_items * a.H, a.dv / DVT);
  // reverse walk first (it starts where the boundary pass ended and ends
  // where the dq walk starts: both begin on rows still in the last-level
  // cache)
  hipLaunchKernelGGL((bwd_dkdv_kernel<DVT, DKT>), dim3(grid), dim3(512), 0, s,
                     (const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.v,
                     (const bf16 *)a.dout, a.ds_final, a.cslots, (bf16 *)a.dv_out,
                     a.ds0, a.part_dk, p, dec, a.scale, a.H, a.dv);
  hipLaunchKernelGGL((bwd_dq_kernel<DVT, DKT>), dim3(grid), dim3(512), 0, s,
                     (const bf16 *)a.k, (const bf16 *)a.v, (const bf16 *)a.dout,
                     a.s0, a.slots, a.part_dq, p, dec, a.scale, a.H, a.dv);
}

hipError_t launch_bwd_mfma(int dvt, const Plan &p, const BwdArgs &a,
                           const Decay &dec, hipStream_t s) {
  if (a.dk_dim == 64) launch_bwd_dvt<64, 64>(p, a, dec, s);
  else if (a.dk_dim == 128) launch_bwd_dvt<64, 128>(p, a, dec, s);
  else if (dvt == 96) launch_bwd_dvt<96, 96>(p, a, dec, s);
  else launch_bwd_dvt<64, 96>(p, a, dec, s);
  const long long n4 = (long long)p.total_T * a.H * (a.dk_dim / 4);
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s,
                     a.part_dq, a.part_dk, (bf16 *)a.dq, (bf16 *)a.dk, (long long)p.total_T,
                     a.H, a.dv / dvt, a.dk_dim);
  return hipGetLastError();
}

}  // namespace gla
