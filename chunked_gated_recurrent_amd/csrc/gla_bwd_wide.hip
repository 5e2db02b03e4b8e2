// gla_bwd_wide.hip -- backward of the chunked Simple GLA forward for bf16
// inputs with dk 64, 96 or 128 and dv 64, 128 or 192 (the Laplace 3B head:
// dk 96, dv 192; not dk 128 with dv 192, whose tiles exceed the LDS), one
// workgroup per (work item, head) owning all value columns.
//
// Same gradients and chunk formulas as gla_bwd_mfma.hip (Laplace 3B /
// Trainium2 page, sections "GLA mixer" and "Challenge 3"). There, dq and dk
// contract over dv split into two tiles and leave fp32 partial rows for a
// third pass to add (about 0.8 GB of extra traffic at the Laplace batch);
// here a workgroup holds the whole dv, so dq and dk come out complete and
// go straight to their bf16 rows. The price is LDS: the tiles of a chunk
// (at dv 192, 125 KB in the dq pass and 140 KB in the reverse walk; 94 and
// 109 KB at dv 128) fit only once, so
// every chunk takes two barriers (tiles and published state ready / all
// reads done) instead of double buffers, and one workgroup per CU does.
// When the batch's (sequence, head) units with two workgroups each fill
// the GPU, both walks run in one launch (bwd_fused_wide_kernel); otherwise
// the planner cuts sequences into time segments and the walks run one
// after the other.
//
//   bwd_dq_wide_kernel   forward walk. Waves 0-3 ("dq waves", rows 16 w ..
//                        16 w + 15 of each chunk) form dq; waves 4-7 rebuild
//                        S (a 3 x dv/32 block of 16 x 16 tiles each) and
//                        publish its bf16 transpose every chunk.
//   bwd_dkdv_wide_kernel reverse walk. Waves 0-3 form dv, waves 4-7 dk, and
//                        each wave also advances a 3 x dv/64 block of tiles
//                        of the carried gradient Ch (the first half of the
//                        column tiles on the dv waves, the second on the dk
//                        waves), published as bf16 Ch^T every chunk.
//   bwd_fused_wide_kernel both walks in one launch, the dq walk's
//                        workgroups also forming the dk and dv rows of each
//                        sequence's last chunks.
// Outputs are written from registers: each lane stores the 4 consecutive
// values of one row that an MFMA result tile gives it (8-byte stores).
#include "gla_mfma.h"

namespace gla {

namespace {

// LDS of the reverse walk (the larger pass): q, scaled q and k tiles, v and
// dO tiles, the published Ch^T and the decay powers.
constexpr int wide_lds(int dk, int dv) {
  return 64 * (dk + 16) * 2 * 3 + 64 * (dv + 16) * 2 * 2 + dv * (dk + 16) * 2 + 4 * 68;
}
// The head shapes these kernels take: each reverse wave owns a quarter of
// the column tiles of Ch, and the reverse walk's tiles must fit the LDS
// (dk 128 with dv 192 does not).
constexpr bool wide_shape(int dk, int dv) {
  return (dk == 64 || dk == 96 || dk == 128) && (dv == 64 || dv == 128 || dv == 192) &&
         wide_lds(dk, dv) <= 160 * 1024;
}

// Per-shape constants, declared inside every templated function; at dk 96,
// dv 192: C 64, QS 112, VS 208, NCT 12, NDT 6.
#define WIDE_CONSTS(DK_, DV_)                                                 \
  using MW = MfCfg<DV_, DK_>;                                                 \
  [[maybe_unused]] constexpr int kWideDv = DV_;                               \
  [[maybe_unused]] constexpr int kWC = MW::C, kWQS = MW::QS, kWVS = MW::VS;   \
  [[maybe_unused]] constexpr int kWNCS = DV_ / 32; /* 32-deep steps over dv */ \
  static_assert(wide_shape(DK_, DV_), "head shape of the wide backward")

// The state S^T published by the dq pass's state waves keeps its 8-column
// blocks XOR-swizzled by bit 3 of the row: element (c, d) sits at
// c * QS + (d ^ (c & 8)). Its only readers are transposing reads of aligned
// 4-column groups, which the swizzle keeps whole; it halves the LDS bank
// conflicts of the publish (16 rows written at one column offset).
__device__ __forceinline__ int swz8(int r, int c) { return c ^ (r & 8); }

// A compile-time switch passed to generic lambdas (`if constexpr` on it).
template <bool B>
struct Flag {
  static constexpr bool value = B;
};

// One tile load pattern: `n` 16-byte vectors per role thread over a chunk
// tile of `per_row` vectors per row.
template <int N>
struct TileIdx {
  int row[N], col[N];
  __device__ __forceinline__ TileIdx(int rt, int per_row) {
#pragma unroll
    for (int m = 0; m < N; ++m) {
      const int vi = rt + 256 * m;
      row[m] = vi / per_row;
      col[m] = vi - row[m] * per_row;
    }
  }
};

}  // namespace

// ---------------------------------------------------------------------------
// dq pass
// ---------------------------------------------------------------------------
template <int DKT, int DV>
__device__ __forceinline__ void wide_dq_role(
    const bf16 *__restrict__ dout, bf16 *__restrict__ dq, const Item &it, int h, int H,
    float scale, int rt, int w, bf16 *sD, const bf16 *sK, const bf16 *sV, const bf16 *sSt,
    const float *sPow) {
  WIDE_CONSTS(DKT, DV);
  constexpr int C = kWC, QS = kWQS, VS = kWVS, VV = MW::VV, NDT = MW::NDT, NJS = MW::NJS;
  const int lane = rt & 63, l16 = lane & 15, g = lane >> 4;
  const int tr_row = l16 >> 2, tr_col = 4 * (l16 & 3);
  const unsigned rowVb = (unsigned)(H * kWideDv * 2);
  const int nch = (it.t1 - it.t0 + C - 1) / C;
  const TileIdx<VV> ix(rt, MW::NVV);

  auto load = [&](int ch, u32x4(&r)[VV]) {
    const long long tb = (long long)it.t0 + (long long)ch * C;
    const __amdgpu_buffer_rsrc_t bd =
        buf_rsrc(dout + tb * H * kWideDv + (long long)h * kWideDv,
                 (unsigned)chunk_rows(it, ch) * rowVb);
#pragma unroll
    for (int m = 0; m < VV; ++m)
      r[m] = __builtin_amdgcn_raw_buffer_load_b128(bd, ix.row[m] * rowVb + ix.col[m] * 16, 0, 0);
  };
  auto store = [&](const u32x4(&r)[VV]) {
#pragma unroll
    for (int m = 0; m < VV; ++m)
      *reinterpret_cast<u32x4 *>(sD + ix.row[m] * VS + 8 * ix.col[m]) = r[m];
  };

  u32x4 ra[VV], rb[VV];
  load(0, ra);
  load(1, rb);
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
  store(ra);

  auto body = [&](int ch, u32x4(&rnew)[VV], const u32x4(&rnext)[VV]) {
    __syncthreads();  // A: chunk ch and S_{ch-1} are in LDS
    load(ch + 2, rnew);
    bf16x8 dfn[kWNCS], dfp[kWNCS];  // dO row i: natural and P k-sets over dv
#pragma unroll
    for (int s = 0; s < kWNCS; ++s) {
      const int row = i_row * VS + 32 * s;
      dfn[s] = *reinterpret_cast<const bf16x8 *>(sD + row + 8 * g);
      dfp[s] = cat8(lds8_apart(sD, row + 4 * g), lds8_apart(sD, row + 16 + 4 * g));
    }
    // P'^T[j][i] = v_j . dO_i over all of dv, j blocks 0..3
    f32x4 p[4];
#pragma unroll
    for (int J = 0; J < 4; ++J) p[J] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kWNCS; ++s)
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        const bf16x8 vfr = *reinterpret_cast<const bf16x8 *>(sV + (16 * J + l16) * VS + 32 * s + 8 * g);
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
    for (int s = 0; s < kWNCS; ++s)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int row = 32 * s + 4 * g + tr_row;  // row + 16 has the same bit 3
        const bf16 *base = sSt + row * QS + swz8(row, 16 * dt + tr_col);
        acc[dt] = mfma(cat8(tr4(base), tr4(base + 16 * QS)), dfp[s], acc[dt]);
      }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[dt] *= lam_i1;
#pragma unroll
    for (int s = 0; s < NJS; ++s)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const bf16 *base = sK + (32 * s + 4 * g + tr_row) * QS + 16 * dt + tr_col;
        acc[dt] = mfma(cat8(tr4(base), tr4(base + 16 * QS)), pb[s], acc[dt]);
      }
    {  // dq row i: this lane holds dk values 16 dt + 4 g .. + 3 (rows past
       // the item's end fall outside the descriptor)
      const unsigned rowKb = (unsigned)(H * DKT * 2);
      const __amdgpu_buffer_rsrc_t bo =
          buf_rsrc(dq + ((it.t0 + (long long)ch * C) * H + h) * DKT,
                   (unsigned)chunk_rows(it, ch) * rowKb);
      const unsigned o0 = (unsigned)i_row * rowKb + 8 * g;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        bf16x4 t;
#pragma unroll
        for (int r = 0; r < 4; ++r) t[r] = (bf16)(scale * acc[dt][r]);
        buf_store8(t, bo, o0 + 32 * dt);
      }
    }
    // keep the result tiles' registers from living on into what follows
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();  // B: every read of chunk ch and S_{ch-1} is done
    store(rnext);
  };
  for (int ch = 0; ch < nch; ch += 2) {  // a past-the-end chunk is all zeros
    body(ch, ra, rb);
    body(ch + 1, rb, ra);
  }
}

// With `pair` set (every sequence is cut into exactly two segments and the
// slots hold the raw local quantities, not yet scanned), the incoming value
// of the second segment is formed here: U_0 + lambda^len0 S0.
template <int DKT, int DV>
__device__ __forceinline__ void wide_state_role(
    const bf16 *__restrict__ k, const bf16 *__restrict__ v, const float *__restrict__ s0,
    const float *__restrict__ slots, const Item &it, int idx, int h, int H, int rt, int w,
    bf16 *sK, bf16 *sKs, bf16 *sV, bf16 *sSt, const float *sPow, const float *pair_add,
    float pair_scale) {
  WIDE_CONSTS(DKT, DV);
  constexpr int C = kWC, DK = DKT, QS = kWQS, VS = kWVS, QV = MW::QV, VV = MW::VV;
  constexpr int SDT = MW::SDT, SCT = MW::SCT, NJS = MW::NJS;
  const int lane = rt & 63, l16 = lane & 15, g = lane >> 4;
  const int tr_row = l16 >> 2, tr_col = 4 * (l16 & 3);
  const unsigned rowKb = (unsigned)(H * DK * 2), rowVb = (unsigned)(H * kWideDv * 2);
  const int nch = (it.t1 - it.t0 + C - 1) / C;
  const int dt0 = SDT * (w >> 1), ct0 = SCT * (w & 1);
  const TileIdx<QV> ik(rt, MW::NQV);
  const TileIdx<VV> iv(rt, MW::NVV);

  f32x4 accS[SDT][SCT];
  {
    const float *src = (it.flags & kFirstSeg)
                           ? (s0 ? s0 + ((long long)it.n * H + h) * DK * kWideDv : nullptr)
                           : slots + ((long long)(idx - 1) * H + h) * DK * kWideDv;
#pragma unroll
    for (int a = 0; a < SDT; ++a)
#pragma unroll
      for (int b = 0; b < SCT; ++b) {
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
        const int d = 16 * (dt0 + a) + 4 * g;
        const int c = 16 * (ct0 + b) + l16;
        if (src) {
#pragma unroll
          for (int r = 0; r < 4; ++r) x[r] = src[(long long)(d + r) * kWideDv + c];
        }
        if (pair_add) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            x[r] = fmaf(pair_scale, pair_add[(long long)(d + r) * kWideDv + c], x[r]);
        }
        accS[a][b] = x;
      }
  }
  auto load = [&](int ch, u32x4(&rk)[QV], u32x4(&rv)[VV]) {
    const long long tb = (long long)it.t0 + (long long)ch * C;
    const unsigned L = (unsigned)chunk_rows(it, ch);
    const __amdgpu_buffer_rsrc_t bk = buf_rsrc(k + (tb * H + h) * DK, L * rowKb);
    const __amdgpu_buffer_rsrc_t bv = buf_rsrc(v + (tb * H + h) * kWideDv, L * rowVb);
#pragma unroll
    for (int m = 0; m < QV; ++m)
      rk[m] = __builtin_amdgcn_raw_buffer_load_b128(bk, ik.row[m] * rowKb + ik.col[m] * 16, 0, 0);
#pragma unroll
    for (int m = 0; m < VV; ++m)
      rv[m] = __builtin_amdgcn_raw_buffer_load_b128(bv, iv.row[m] * rowVb + iv.col[m] * 16, 0, 0);
  };
  auto store = [&](int L, const u32x4(&rk)[QV], const u32x4(&rv)[VV]) {
#pragma unroll
    for (int m = 0; m < QV; ++m) {
      const int r = ik.row[m];
      *reinterpret_cast<u32x4 *>(sK + r * QS + 8 * ik.col[m]) = rk[m];
      // decay-scaled copy lambda^(L-1-r) k_r; rows past the end are zero
      const float wgt = r < L ? sPow[max(L - 1 - r, 0)] : 0.f;
      const bf16x8 kv = __builtin_bit_cast(bf16x8, rk[m]);
      bf16x8 ks;
#pragma unroll
      for (int e = 0; e < 8; ++e) ks[e] = (bf16)((float)kv[e] * wgt);
      *reinterpret_cast<bf16x8 *>(sKs + r * QS + 8 * ik.col[m]) = ks;
    }
#pragma unroll
    for (int m = 0; m < VV; ++m)
      *reinterpret_cast<u32x4 *>(sV + iv.row[m] * VS + 8 * iv.col[m]) = rv[m];
  };
  auto publish = [&]() {  // S^T as bf16: row c, columns d
#pragma unroll
    for (int a = 0; a < SDT; ++a)
#pragma unroll
      for (int b = 0; b < SCT; ++b) {
        bf16x4 t;
#pragma unroll
        for (int r = 0; r < 4; ++r) t[r] = (bf16)accS[a][b][r];
        const int c = 16 * (ct0 + b) + l16;
        *reinterpret_cast<bf16x4 *>(sSt + c * QS + swz8(c, 16 * (dt0 + a) + 4 * g)) = t;
      }
  };

  u32x4 ka[QV], kb[QV], va[VV], vb[VV];
  load(0, ka, va);
  load(1, kb, vb);
  __syncthreads();  // sPow ready
  store(chunk_rows(it, 0), ka, va);
  publish();  // S_{-1}: the incoming state

  auto body = [&](int ch, u32x4(&kn)[QV], u32x4(&vn)[VV], const u32x4(&kx)[QV],
                  const u32x4(&vx)[VV]) {
    const int L = chunk_rows(it, ch);
    __syncthreads();  // A: chunk ch and S_{ch-1} are in LDS
    load(ch + 2, kn, vn);
    const float lamL = sPow[L];
#pragma unroll
    for (int a = 0; a < SDT; ++a)
#pragma unroll
      for (int b = 0; b < SCT; ++b) accS[a][b] *= lamL;
#pragma unroll
    for (int s = 0; s < NJS; ++s) {
      bf16x8 af[SDT], bfr[SCT];
      const int row = 32 * s + 4 * g + tr_row;
#pragma unroll
      for (int a = 0; a < SDT; ++a) {
        const bf16 *base = sKs + row * QS + 16 * (dt0 + a) + tr_col;
        af[a] = cat8(tr4(base), tr4(base + 16 * QS));
      }
#pragma unroll
      for (int b = 0; b < SCT; ++b) {
        const bf16 *base = sV + row * VS + 16 * (ct0 + b) + tr_col;
        bfr[b] = cat8(tr4(base), tr4(base + 16 * VS));
      }
#pragma unroll
      for (int a = 0; a < SDT; ++a)
#pragma unroll
        for (int b = 0; b < SCT; ++b) accS[a][b] = mfma(af[a], bfr[b], accS[a][b]);
    }
    __syncthreads();  // B: every read of chunk ch and S_{ch-1} is done
    store(chunk_rows(it, ch + 1), kx, vx);
    publish();  // S_ch for the next chunk's dq rows
  };
  for (int ch = 0; ch < nch; ch += 2) {
    body(ch, ka, va, kb, vb);
    body(ch + 1, kb, vb, ka, va);
  }
}

// LDS of the two walks (bytes, 16-byte multiples): the dq walk holds k, its
// decay-scaled copy, v, dO and the published S^T; the reverse walk q, its
// decay-scaled copy, k, v, dO and the published Ch^T; both the decay powers.
template <int DKT, int DV>
struct WideLds {
  static constexpr int QT = 64 * (DKT + 16) * 2, VT = 64 * (DV + 16) * 2;
  static constexpr int ST = DV * (DKT + 16) * 2, POW = 68 * 4;
  static constexpr int DQ = 2 * QT + 2 * VT + ST + POW;
  static constexpr int REV = 3 * QT + 2 * VT + ST + POW;
  static constexpr int MAX = DQ > REV ? DQ : REV;
};

// The dq walk of the workgroup with id P in its walk's grid (see
// bwd_dq_wide_kernel), on the LDS block `lds`.
template <int DKT, int DV>
__device__ __forceinline__ void dq_wide_walk(
    const bf16 *__restrict__ k, const bf16 *__restrict__ v, const bf16 *__restrict__ dout,
    const float *__restrict__ s0, const float *__restrict__ slots, bf16 *__restrict__ dq,
    const Plan &plan, const Decay &dec, float scale, int H, int pair, int P, char *lds) {
  WIDE_CONSTS(DKT, DV);
  using LD = WideLds<DKT, DV>;
  bf16 *sK = (bf16 *)lds;
  bf16 *sKs = (bf16 *)(lds + LD::QT);
  bf16 *sV = (bf16 *)(lds + 2 * LD::QT);
  bf16 *sD = (bf16 *)(lds + 2 * LD::QT + LD::VT);
  bf16 *sSt = (bf16 *)(lds + 2 * LD::QT + 2 * LD::VT);
  float *sPow = (float *)(lds + 2 * LD::QT + 2 * LD::VT + LD::ST);

  int unit, dtile;
  xcd_unit_at(plan, P, 1, plan.max_items * H, unit, dtile);
  if (unit >= plan.max_items * H) return;
  const int slot = unit / H;
  const int h = unit - slot * H;
  int idx;
  Item it;
  if (!slot_item(plan, slot, idx, it)) return;
  make_uniform(idx, it);
  const int tid = threadIdx.x;
  if (tid <= kWC) sPow[tid] = pow_f64(dec.lam[h], tid);
  const int role_wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (role_wave < 4) {
    wide_dq_role<DKT, DV>(dout, dq, it, h, H, scale, tid & 255, role_wave, sD, sK, sV, sSt, sPow);
  } else {
    const float *pair_add = nullptr;
    float pair_scale = 0.f;
    if (pair && !(it.flags & kFirstSeg) && s0) {  // second of two segments
      Item prev;
      load_item(plan, idx - 1, prev);
      pair_add = s0 + ((long long)it.n * H + h) * DKT * DV;
      pair_scale = pow_f64(dec.lam[h], prev.t1 - prev.t0);
    }
    wide_state_role<DKT, DV>(k, v, s0, slots, it, idx, h, H, tid & 255, role_wave - 4, sK, sKs, sV,
                    sSt, sPow, pair_add, pair_scale);
  }
}

template <int DKT, int DV>
__global__ __launch_bounds__(512, 1) void bwd_dq_wide_kernel(
    const bf16 *__restrict__ k, const bf16 *__restrict__ v, const bf16 *__restrict__ dout,
    const float *__restrict__ s0, const float *__restrict__ slots, bf16 *__restrict__ dq,
    Plan plan, Decay dec, float scale, int H, int pair) {
  __shared__ __attribute__((aligned(16))) char lds[WideLds<DKT, DV>::DQ];
  dq_wide_walk<DKT, DV>(k, v, dout, s0, slots, dq, plan, dec, scale, H, pair, (int)blockIdx.x,
                        lds);
}

// ---------------------------------------------------------------------------
// Reverse walk: dv and dk rows, Ch split over both roles
// ---------------------------------------------------------------------------
template <int DKT, int DV, bool DV_ROLE>
__device__ __forceinline__ void wide_rev_role(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const bf16 *__restrict__ dout, const float *__restrict__ ds_final,
    const float *__restrict__ cslots, bf16 *__restrict__ out, float *__restrict__ ds0,
    const Item &it, int idx, int h, int H, float scale, int rt, int w, bf16 *sQ, bf16 *sQs,
    bf16 *sK, bf16 *sV, bf16 *sD, bf16 *sCt, const float *sPow, const float *pair_add,
    float pair_scale, int n_out) {
  WIDE_CONSTS(DKT, DV);
  constexpr int C = kWC, DK = DKT, QS = kWQS, VS = kWVS, QV = MW::QV, VV = MW::VV;
  constexpr int NDT = MW::NDT, NCT = MW::NCT, NJS = MW::NJS, NKS = MW::NKS;
  // loads per role thread and register stage: the dv role brings q and k
  // (QV each) and dO rows 0-31 (ND), the dk role v (VV) and dO rows 32-63
  // (ND); at d_v 192 that is 9 vectors for either role
  constexpr int ND = 32 * MW::NVV / 256;
  constexpr int NA = DV_ROLE ? QV : VV;  // q then k, or v
  constexpr int NL = (DV_ROLE ? 2 * QV : VV) + ND;
  // Ch: each wave owns RB d tiles (half of them) x CB column tiles (a
  // quarter of them)
  constexpr int RB = NDT / 2, CB = NCT / 4;
  static_assert(NDT % 2 == 0 && NCT % 4 == 0 && 32 * MW::NVV % 256 == 0, "reverse split");
  const int lane = rt & 63, l16 = lane & 15, g = lane >> 4;
  const int tr_row = l16 >> 2, tr_col = 4 * (l16 & 3);
  const unsigned rowKb = (unsigned)(H * DK * 2), rowVb = (unsigned)(H * kWideDv * 2);
  const int nch = (it.t1 - it.t0 + C - 1) / C;
  const int i_row = 16 * w + l16;
  const long long state_off = ((long long)it.n * H + h) * DK * kWideDv;
  const TileIdx<NA> ia(rt, DV_ROLE ? MW::NQV : MW::NVV);
  const TileIdx<ND> idh(rt, MW::NVV);  // rows 0-31 of the dO tile
  const int drow0 = DV_ROLE ? 0 : 32;
  auto rows_of = [&](int ch) { return ch < 0 ? 0 : chunk_rows(it, ch); };

  // A chunk from n_out on only carries the gradient, which needs its q and
  // dO alone: `kv` false leaves out the k and v tiles (their loads and LDS
  // stores; the slots of r they would fill stay unused). Which chunks get
  // which form is fixed by the straight-line code around each call, so the
  // compiler's waits on the loads stay exact (a branch around loads makes
  // every later wait assume they were skipped and wait for newer loads too).
  // A k or v load of a chunk at or past n_out gets an empty descriptor and
  // reads zeros without memory traffic.
  auto load_kv = [&](auto kv, int ch, u32x4(&r)[NL]) {
    const unsigned L = (unsigned)rows_of(ch);
    const unsigned Lkv = ch < n_out ? L : 0u;
    const long long tb = (long long)it.t0 + (long long)(ch < 0 ? 0 : ch) * C;
    const __amdgpu_buffer_rsrc_t bd = buf_rsrc(dout + (tb * H + h) * kWideDv, L * rowVb);
    if (DV_ROLE) {
      const __amdgpu_buffer_rsrc_t bq = buf_rsrc(q + (tb * H + h) * DK, L * rowKb);
#pragma unroll
      for (int m = 0; m < QV; ++m)
        r[m] = __builtin_amdgcn_raw_buffer_load_b128(bq, ia.row[m] * rowKb + ia.col[m] * 16, 0, 0);
      if constexpr (decltype(kv)::value) {
        const __amdgpu_buffer_rsrc_t bk = buf_rsrc(k + (tb * H + h) * DK, Lkv * rowKb);
#pragma unroll
        for (int m = 0; m < QV; ++m)
          r[QV + m] = __builtin_amdgcn_raw_buffer_load_b128(bk, ia.row[m] * rowKb + ia.col[m] * 16, 0, 0);
      }
    } else if constexpr (decltype(kv)::value) {
      const __amdgpu_buffer_rsrc_t bv = buf_rsrc(v + (tb * H + h) * kWideDv, Lkv * rowVb);
#pragma unroll
      for (int m = 0; m < VV; ++m)
        r[m] = __builtin_amdgcn_raw_buffer_load_b128(bv, ia.row[m] * rowVb + ia.col[m] * 16, 0, 0);
    }
#pragma unroll
    for (int m = 0; m < ND; ++m)
      r[NL - ND + m] = __builtin_amdgcn_raw_buffer_load_b128(
          bd, (drow0 + idh.row[m]) * rowVb + idh.col[m] * 16, 0, 0);
  };
  auto load = [&](int ch, u32x4(&r)[NL]) { load_kv(Flag<true>{}, ch, r); };
  float fqr[NA];  // dv role: scale * lambda^(t+1) of the q rows this thread stores
  auto store_kv = [&](auto kv, const u32x4(&r)[NL]) {
    if (DV_ROLE) {
#pragma unroll
      for (int m = 0; m < QV; ++m) {
        if constexpr (decltype(kv)::value) {
          *reinterpret_cast<u32x4 *>(sQ + ia.row[m] * QS + 8 * ia.col[m]) = r[m];
          *reinterpret_cast<u32x4 *>(sK + ia.row[m] * QS + 8 * ia.col[m]) = r[QV + m];
        }
        // the carry's decay-scaled copy of q, made once per chunk
        const bf16x8 qv = __builtin_bit_cast(bf16x8, r[m]);
        bf16x8 qs;
#pragma unroll
        for (int e = 0; e < 8; ++e) qs[e] = (bf16)((float)qv[e] * fqr[m]);
        *reinterpret_cast<bf16x8 *>(sQs + ia.row[m] * QS + 8 * ia.col[m]) = qs;
      }
    } else if constexpr (decltype(kv)::value) {
#pragma unroll
      for (int m = 0; m < VV; ++m)
        *reinterpret_cast<u32x4 *>(sV + ia.row[m] * VS + 8 * ia.col[m]) = r[m];
    }
#pragma unroll
    for (int m = 0; m < ND; ++m)
      *reinterpret_cast<u32x4 *>(sD + (drow0 + idh.row[m]) * VS + 8 * idh.col[m]) = r[NL - ND + m];
  };
  auto store = [&](const u32x4(&r)[NL]) { store_kv(Flag<true>{}, r); };

  // this wave's RB x CB tiles of the carried gradient Ch: d tiles dt0..,
  // column tiles ct0.. (the first half on the dv role, the second half on
  // the dk role; 0-5 and 6-11 at d_v 192). Ch starts as
  // dL/dS_final for a sequence's last item, else as the combined carry
  // flowing out of the next item (its slot)
  const int dt0 = RB * (w >> 1), ct0 = (DV_ROLE ? 0 : NCT / 2) + CB * (w & 1);
  const float *cin = (it.flags & kLastSeg)
                         ? (ds_final ? ds_final + state_off : nullptr)
                         : cslots + ((long long)(idx + 1) * H + h) * DK * kWideDv;
  f32x4 accC[RB][CB];
#pragma unroll
  for (int a = 0; a < RB; ++a)
#pragma unroll
    for (int b = 0; b < CB; ++b) {
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
      const int d = 16 * (dt0 + a) + 4 * g;
      const int c = 16 * (ct0 + b) + l16;
      if (cin) {
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = cin[(long long)(d + r) * kWideDv + c];
      }
      if (pair_add) {  // first of two segments: U'_1 + lambda^len1 dL/dS_final
#pragma unroll
        for (int r = 0; r < 4; ++r)
          x[r] = fmaf(pair_scale, pair_add[(long long)(d + r) * kWideDv + c], x[r]);
      }
      accC[a][b] = x;
    }
  auto publish = [&]() {  // Ch^T as bf16, row c, columns d
#pragma unroll
    for (int a = 0; a < RB; ++a)
#pragma unroll
      for (int b = 0; b < CB; ++b) {
        bf16x4 t;
#pragma unroll
        for (int r = 0; r < 4; ++r) t[r] = (bf16)accC[a][b][r];
        const int c = 16 * (ct0 + b) + l16;
        *reinterpret_cast<bf16x4 *>(sCt + c * QS + 16 * (dt0 + a) + 4 * g) = t;
      }
  };

  u32x4 ra[NL], rb[NL];
  load(nch - 1, ra);
  load(nch - 2, rb);
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
#pragma unroll
  for (int m = 0; m < NA; ++m) fqr[m] = DV_ROLE ? scale * sPow[ia.row[m] + 1] : 0.f;
  // carry-only chunks: the last nc of the item (an even count); Ch^T is
  // read only by full chunks, so it is published before the first of them
  const int nc = nch - n_out;
  if (nc > 0) {
    store_kv(Flag<false>{}, ra);
  } else {
    store(ra);
    publish();
  }

  // Ch <- lambda^L Ch + scale sum_t lambda^(t+1) q_t^T dO_t (this wave's
  // tiles) over the L rows of the chunk in LDS
  auto advance = [&](int L) {
    const float lamL = sPow[L];
#pragma unroll
    for (int a = 0; a < RB; ++a)
#pragma unroll
      for (int b = 0; b < CB; ++b) accC[a][b] *= lamL;
#pragma unroll
    for (int s = 0; s < NJS; ++s) {
      bf16x8 qa[RB], dfr[CB];  // scale lambda^(t+1) q_t (P k-set over t) and dO
      const int row = 32 * s + 4 * g + tr_row;
#pragma unroll
      for (int a = 0; a < RB; ++a) {
        const bf16 *base = sQs + row * QS + 16 * (dt0 + a) + tr_col;
        qa[a] = cat8(tr4(base), tr4(base + 16 * QS));
      }
#pragma unroll
      for (int b = 0; b < CB; ++b) {
        const bf16 *base = sD + row * VS + 16 * (ct0 + b) + tr_col;
        dfr[b] = cat8(tr4(base), tr4(base + 16 * VS));
      }
#pragma unroll
      for (int a = 0; a < RB; ++a)
#pragma unroll
        for (int b = 0; b < CB; ++b) accC[a][b] = mfma(qa[a], dfr[b], accC[a][b]);
    }
  };

  auto body = [&](int ch, u32x4(&rn)[NL], const u32x4(&rx)[NL]) {
    const int L = rows_of(ch);
    const long long tb = (long long)it.t0 + (long long)(ch < 0 ? 0 : ch) * C;
    __syncthreads();  // A: chunk ch and Ch_in are in LDS
    load(ch - 2, rn);
    const float lam_rev = sPow[clampi(L - 1 - i_row, 0, C)];  // lambda^(L-1-i)
    if (DV_ROLE) {
      // scores A[t][i] = q_t . k_i (natural k-set over d)
      bf16x8 kf[NKS];
#pragma unroll
      for (int s = 0; s < NKS; ++s)
        kf[s] = *reinterpret_cast<const bf16x8 *>(sK + i_row * QS + 32 * s + 8 * g);
      f32x4 sc[4];
#pragma unroll
      for (int T = 0; T < 4; ++T) sc[T] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NKS; ++s)
#pragma unroll
        for (int T = 0; T < 4; ++T) {
          const bf16x8 qf = *reinterpret_cast<const bf16x8 *>(sQ + (16 * T + l16) * QS + 32 * s + 8 * g);
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
          const bf16x8 cf = *reinterpret_cast<const bf16x8 *>(sCt + (16 * ct + l16) * QS + 32 * s + 8 * g);
          acc[ct] = mfma(cf, kf[s], acc[ct]);
        }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) acc[ct] *= lam_rev;
#pragma unroll
      for (int s = 0; s < NJS; ++s)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const bf16 *base = sD + (32 * s + 4 * g + tr_row) * VS + 16 * ct + tr_col;
          acc[ct] = mfma(cat8(tr4(base), tr4(base + 16 * VS)), ab[s], acc[ct]);
        }
      if (i_row < L) {  // dv row i: values 16 ct + 4 g .. + 3
        bf16 *dst = out + ((tb + i_row) * H + h) * kWideDv + 4 * g;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          bf16x4 t;
#pragma unroll
          for (int r = 0; r < 4; ++r) t[r] = (bf16)acc[ct][r];
          *reinterpret_cast<bf16x4 *>(dst + 16 * ct) = t;
        }
      }
    } else {
      // scores Bm[t][i] = dO_t . v_i over dv (natural k-set over c: both
      // operands are 16-byte row reads)
      f32x4 sc[4];
#pragma unroll
      for (int T = 0; T < 4; ++T) sc[T] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < kWNCS; ++s) {
        const bf16x8 vn = *reinterpret_cast<const bf16x8 *>(sV + i_row * VS + 32 * s + 8 * g);
#pragma unroll
        for (int T = 0; T < 4; ++T) {
          const bf16x8 df =
              *reinterpret_cast<const bf16x8 *>(sD + (16 * T + l16) * VS + 32 * s + 8 * g);
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
      for (int s = 0; s < kWNCS; ++s) {
        // v_i in the P k-set over c, matching the transposed reads of Ch
        const int vrow = i_row * VS + 32 * s;
        const bf16x8 vf = cat8(lds8_apart(sV, vrow + 4 * g), lds8_apart(sV, vrow + 16 + 4 * g));
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const bf16 *base = sCt + (32 * s + 4 * g + tr_row) * QS + 16 * dt + tr_col;
          acc[dt] = mfma(cat8(tr4(base), tr4(base + 16 * QS)), vf, acc[dt]);
        }
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) acc[dt] *= lam_rev;
#pragma unroll
      for (int s = 0; s < NJS; ++s)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const bf16 *base = sQ + (32 * s + 4 * g + tr_row) * QS + 16 * dt + tr_col;
          acc[dt] = mfma(cat8(tr4(base), tr4(base + 16 * QS)), bm[s], acc[dt]);
        }
      if (i_row < L) {  // dk row i: values 16 dt + 4 g .. + 3
        bf16 *dst = out + ((tb + i_row) * H + h) * DK + 4 * g;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          bf16x4 t;
#pragma unroll
          for (int r = 0; r < 4; ++r) t[r] = (bf16)acc[dt][r];
          *reinterpret_cast<bf16x4 *>(dst + 16 * dt) = t;
        }
      }
    }
    advance(L);
    __syncthreads();  // B: every read of chunk ch and Ch_in is done
    store(rx);
    publish();
  };
  // chunks from n_out on only carry the gradient back (their dk and dv rows
  // are formed elsewhere): the same update of Ch, nothing else. `kv`: the
  // chunk two ahead (whose loads this one issues) is a full one; `first`:
  // the next chunk is the first full one (full tiles and Ch^T stored)
  auto carry_body = [&](auto kv, auto first, int ch, u32x4(&rn)[NL], const u32x4(&rx)[NL]) {
    __syncthreads();  // A: chunk ch is in LDS
    load_kv(kv, ch - 2, rn);
    advance(rows_of(ch));
    __syncthreads();  // B: every read of chunk ch is done
    if constexpr (decltype(first)::value) {
      store(rx);
      publish();
    } else {
      store_kv(Flag<false>{}, rx);
    }
  };
  // nc is even, so both loops keep the two register stages in turn; the
  // last carry pair issues the loads of the first two full chunks
  int p = 0;
  for (; p + 2 < nc; p += 2) {
    carry_body(Flag<false>{}, Flag<false>{}, nch - 1 - p, ra, rb);
    carry_body(Flag<false>{}, Flag<false>{}, nch - 2 - p, rb, ra);
  }
  if (p < nc) {
    carry_body(Flag<true>{}, Flag<false>{}, nch - 1 - p, ra, rb);
    carry_body(Flag<true>{}, Flag<true>{}, nch - 2 - p, rb, ra);
    p += 2;
  }
  for (; p < nch; p += 2) {  // a chunk before the first is all zeros
    body(nch - 1 - p, ra, rb);
    body(nch - 2 - p, rb, ra);
  }
  // after the first chunk Ch is dL/dS0 (an extra empty step leaves it as is:
  // lambda^0 = 1 and no rows)
  if (ds0 && (it.flags & kFirstSeg)) {
#pragma unroll
    for (int a = 0; a < RB; ++a)
#pragma unroll
      for (int b = 0; b < CB; ++b) {
        const int d = 16 * (dt0 + a) + 4 * g;
        const int c = 16 * (ct0 + b) + l16;
#pragma unroll
        for (int r = 0; r < 4; ++r) ds0[state_off + (long long)(d + r) * kWideDv + c] = accC[a][b][r];
      }
  }
}

// The (item, head) unit of the workgroup with id P in its walk's grid;
// false past the last unit.
__device__ __forceinline__ bool wide_unit(const Plan &plan, int P, int H, int &h, int &idx,
                                          Item &it) {
  int unit, dtile;
  xcd_unit_at(plan, P, 1, plan.max_items * H, unit, dtile);
  if (unit >= plan.max_items * H) return false;
  const int slot = unit / H;
  h = unit - slot * H;
  if (!slot_item(plan, slot, idx, it)) return false;
  make_uniform(idx, it);
  return true;
}

// Chunks at the end of item `it` whose dk and dv rows the dq walk's
// workgroup forms once its own walk is done (see bwd_fused_wide_kernel):
// the share tail_q16 / 65536 of the item's chunks, rounded down to an even
// count and leaving at least one chunk to the reverse walk.
__device__ __forceinline__ int wide_tail_chunks(const Item &it, int tail_q16) {
  const int nch = (it.t1 - it.t0 + 63) / 64;
  const int half = (int)(((long long)nch * tail_q16) >> 17);
  return min(2 * half, (nch - 1) & ~1);
}

// The reverse walk of item `it`, head h, on the LDS block `lds`: dk and dv
// rows of its first n_out chunks (the rest only carry the gradient back).
template <int DKT, int DV>
__device__ __forceinline__ void rev_walk(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const bf16 *__restrict__ dout, const float *__restrict__ ds_final,
    const float *__restrict__ cslots, bf16 *__restrict__ dv_out, bf16 *__restrict__ dk_out,
    float *__restrict__ ds0, const Item &it, int idx, int h, int H, const Decay &dec,
    float scale, const float *pair_add, float pair_scale, int n_out, char *lds) {
  WIDE_CONSTS(DKT, DV);
  using LD = WideLds<DKT, DV>;
  bf16 *sQ = (bf16 *)lds;
  bf16 *sQs = (bf16 *)(lds + LD::QT);
  bf16 *sK = (bf16 *)(lds + 2 * LD::QT);
  bf16 *sV = (bf16 *)(lds + 3 * LD::QT);
  bf16 *sD = (bf16 *)(lds + 3 * LD::QT + LD::VT);
  bf16 *sCt = (bf16 *)(lds + 3 * LD::QT + 2 * LD::VT);
  float *sPow = (float *)(lds + 3 * LD::QT + 2 * LD::VT + LD::ST);
  const int tid = threadIdx.x;
  if (tid <= kWC) sPow[tid] = pow_f64(dec.lam[h], tid);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (wave < 4)
    wide_rev_role<DKT, DV, true>(q, k, v, dout, ds_final, cslots, dv_out, ds0, it, idx, h, H,
                                 scale, tid & 255, wave, sQ, sQs, sK, sV, sD, sCt, sPow,
                                 pair_add, pair_scale, n_out);
  else
    wide_rev_role<DKT, DV, false>(q, k, v, dout, ds_final, cslots, dk_out, ds0, it, idx, h, H,
                                  scale, tid & 255, wave - 4, sQ, sQs, sK, sV, sD, sCt, sPow,
                                  pair_add, pair_scale, n_out);
}

// The reverse walk of the workgroup with id P in its walk's grid (see
// bwd_dkdv_wide_kernel), on the LDS block `lds`; the last
// wide_tail_chunks(tail_q16) chunks of its item only carry the gradient.
template <int DKT, int DV>
__device__ __forceinline__ void dkdv_wide_walk(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const bf16 *__restrict__ dout, const float *__restrict__ ds_final,
    const float *__restrict__ cslots, bf16 *__restrict__ dv_out, bf16 *__restrict__ dk_out,
    float *__restrict__ ds0, const Plan &plan, const Decay &dec, float scale, int H, int pair,
    int tail_q16, int P, char *lds) {
  int h, idx;
  Item it;
  if (!wide_unit(plan, P, H, h, idx, it)) return;
  const float *pair_add = nullptr;
  float pair_scale = 0.f;
  if (pair && !(it.flags & kLastSeg) && ds_final) {  // first of two segments
    Item next;
    load_item(plan, idx + 1, next);
    pair_add = ds_final + ((long long)it.n * H + h) * DKT * DV;
    pair_scale = pow_f64(dec.lam[h], next.t1 - next.t0);
  }
  const int nch = (it.t1 - it.t0 + 63) / 64;
  rev_walk<DKT, DV>(q, k, v, dout, ds_final, cslots, dv_out, dk_out, ds0, it, idx, h, H, dec,
                    scale, pair_add, pair_scale, nch - wide_tail_chunks(it, tail_q16), lds);
}

template <int DKT, int DV>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_wide_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const bf16 *__restrict__ dout, const float *__restrict__ ds_final,
    const float *__restrict__ cslots, bf16 *__restrict__ dv_out, bf16 *__restrict__ dk_out,
    float *__restrict__ ds0, Plan plan, Decay dec, float scale, int H, int pair) {
  __shared__ __attribute__((aligned(16))) char lds[WideLds<DKT, DV>::REV];
  dkdv_wide_walk<DKT, DV>(q, k, v, dout, ds_final, cslots, dv_out, dk_out, ds0, plan, dec, scale,
                          H, pair, 0, (int)blockIdx.x, lds);
}

// Both walks in one launch, for items that are whole sequences (no time
// segments, so no slots): workgroups [0, n_rev) run the reverse walk, the
// rest the dq walk. The walks share nothing, so neither waits on the other,
// and with one workgroup of either kind per CU the batch needs half the
// (sequence, head) units a walk alone needs to fill the GPU.
// A chunk costs the reverse walk more than the dq walk, so the work is
// evened out: the reverse workgroup only carries the gradient back through
// the last wide_tail_chunks(tail_q16) chunks of its sequence (no dk, dv),
// and the dq workgroup first runs a reverse walk over just those chunks,
// starting from dL/dS_final as the sequence's own walk does, then its dq
// walk. Both form every carry with the same operations in the same order,
// so the rows are those of a single walk, bit for bit, and neither
// workgroup waits on the other. Both start on the same last chunks of the
// sequence, on the same XCD, so some of the q and dO rows the carry needs
// come from that XCD's L2 for the second reader (the carry-only pass,
// which loads and stores only q and dO, runs several times as fast, so the
// two drift apart within a few chunks).
// (slots, cslots and pair are the separate kernels' arguments; a plan
// without segments never reads them.)
template <int DKT, int DV>
__global__ __launch_bounds__(512, 1) void bwd_fused_wide_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const bf16 *__restrict__ dout, const float *__restrict__ s0,
    const float *__restrict__ ds_final, const float *__restrict__ slots,
    const float *__restrict__ cslots, bf16 *__restrict__ dq, bf16 *__restrict__ dv_out,
    bf16 *__restrict__ dk_out, float *__restrict__ ds0, Plan plan, Decay dec, float scale,
    int H, int pair, int n_rev, int tail_q16) {
  __shared__ __attribute__((aligned(16))) char lds[WideLds<DKT, DV>::MAX];
  // n_rev is a multiple of 8, so both walks keep the id -> XCD dealing
  if ((int)blockIdx.x < n_rev) {
    dkdv_wide_walk<DKT, DV>(q, k, v, dout, ds_final, cslots, dv_out, dk_out, ds0, plan, dec,
                            scale, H, pair, tail_q16, (int)blockIdx.x, lds);
    return;
  }
  const int P = (int)blockIdx.x - n_rev;
  int h, idx;
  Item it;
  if (!wide_unit(plan, P, H, h, idx, it)) return;
  const int tail = (it.flags & kLastSeg) ? wide_tail_chunks(it, tail_q16) : 0;
  if (tail > 0) {
    // the last `tail` chunks as an item of their own: its walk starts from
    // dL/dS_final and leaves dL/dS0 to the sequence's reverse workgroup
    Item t = it;
    t.t0 = it.t0 + (((it.t1 - it.t0 + 63) / 64) - tail) * 64;
    t.flags = kLastSeg;
    rev_walk<DKT, DV>(q, k, v, dout, ds_final, cslots, dv_out, dk_out, nullptr, t, idx, h, H,
                      dec, scale, nullptr, 0.f, tail, lds);
    __syncthreads();  // every wave is done with the reverse walk's LDS
  }
  dq_wide_walk<DKT, DV>(k, v, dout, s0, slots, dq, plan, dec, scale, H, pair, P, lds);
}

bool bwd_wide_ok(int dk, int dv) { return wide_shape(dk, dv); }

// One head shape; see launch_bwd_wide.
// The reverse walk runs first: it starts at the segments' last rows, which
// the boundary pass read last, and ends at their first rows, where the dq
// walk starts, so both walks begin on rows still in the last-level cache.
template <int DKT, int DV>
static void launch_wide(const Plan &p, const BwdArgs &a, const Decay &dec, int pair,
                           hipStream_t s) {
  const unsigned grid = xcd_grid(p.deal, (long long)p.max_items * a.H, 1);
  hipLaunchKernelGGL((bwd_dkdv_wide_kernel<DKT, DV>), dim3(grid), dim3(512), 0, s, (const bf16 *)a.q,
                     (const bf16 *)a.k, (const bf16 *)a.v, (const bf16 *)a.dout, a.ds_final,
                     a.cslots, (bf16 *)a.dv_out, (bf16 *)a.dk, a.ds0, p, dec, a.scale, a.H,
                     pair);
  hipLaunchKernelGGL((bwd_dq_wide_kernel<DKT, DV>), dim3(grid), dim3(512), 0, s, (const bf16 *)a.k,
                     (const bf16 *)a.v, (const bf16 *)a.dout, a.s0, a.slots, (bf16 *)a.dq, p,
                     dec, a.scale, a.H, pair);
}

template <int DKT, int DV>
static void launch_fused(const Plan &p, const BwdArgs &a, const Decay &dec, int tail_q16,
                         hipStream_t s) {
  const unsigned g = xcd_grid(p.deal, (long long)p.max_items * a.H, 1);
  hipLaunchKernelGGL((bwd_fused_wide_kernel<DKT, DV>), dim3(2 * g), dim3(512), 0, s,
                     (const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.v,
                     (const bf16 *)a.dout, a.s0, a.ds_final, a.slots, a.cslots, (bf16 *)a.dq,
                     (bf16 *)a.dv_out, (bf16 *)a.dk, a.ds0, p, dec, a.scale, a.H, 0, (int)g,
                     tail_q16);
}

// pair: the segment slots hold unscanned local quantities and every sequence
// has exactly two segments (the kernels join them on load). fused: no time
// segments; both walks in one launch, the dq walk's workgroups taking the
// dk and dv rows of the share tail_q16 / 65536 of each sequence's chunks.
hipError_t launch_bwd_wide(const Plan &p, const BwdArgs &a, const Decay &dec, int pair,
                           bool fused, int tail_q16, hipStream_t s) {
  // the shapes wide_shape() admits
#define GLA_WIDE(DK_, DV_)                                     \
  case DK_ * 1000 + DV_:                                       \
    if (fused) launch_fused<DK_, DV_>(p, a, dec, tail_q16, s); \
    else launch_wide<DK_, DV_>(p, a, dec, pair, s);            \
    break;
  switch (a.dk_dim * 1000 + a.dv) {
    GLA_WIDE(96, 192)
    GLA_WIDE(96, 128)
    GLA_WIDE(96, 64)
    GLA_WIDE(64, 192)
    GLA_WIDE(64, 128)
    GLA_WIDE(64, 64)
    GLA_WIDE(128, 128)
    GLA_WIDE(128, 64)
    default: return hipErrorInvalidValue;
  }
#undef GLA_WIDE
  return hipGetLastError();
}

}  // namespace gla
