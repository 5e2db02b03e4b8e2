// gla_mfma.h -- device pieces shared by the chunked kernels on the gfx950
// matrix cores: buffer descriptors, the LDS transpose read, the MFMA wrapper,
// the tile configuration and the state role (the chunk-by-chunk walk of one
// state tile, used by the forward and by the backward's dq pass).
//
// Conventions (see gla_fwd_mfma.hip for the derivation):
//   MFMA lane layout (lane l, l16 = l % 16, g = l / 16): A row l16 and B
//   column l16 with the same 8 k-values for lane group g; D rows 4g..4g+3,
//   column l16. The D layout of two 16 x 16 tiles over k blocks (2s, 2s+1) is
//   a B operand over the k-set {32s + 4g + r, 32s + 16 + 4g + r} (the
//   "P k-set"); an A operand read with ds_read_b64_tr_b16 from a row-major
//   tile whose rows run along k uses the same k-set.
#pragma once

#include "gla_device.h"

namespace gla {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Raw buffer resource (gfx9 family descriptor word 3) over `bytes` bytes.
// Callers pass workgroup-uniform values; reading them back through
// readfirstlane puts the descriptor in scalar registers (a descriptor the
// compiler must treat as per-lane costs a loop around every access).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *base,
                                                           unsigned bytes) {
  const unsigned long long a = (unsigned long long)base;
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)a);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(a >> 32));
  void *p = (void *)(((unsigned long long)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, 0,
                                           (int)__builtin_amdgcn_readfirstlane(bytes),
                                           0x00020000);
}

// Four bf16 (8 bytes) stored at byte offset `off` through a buffer
// descriptor: the hardware drops a store whose offset lies past the
// descriptor's range. Rows past an item's end are skipped this way rather
// than by a branch around the stores, because the wait the compiler places
// before a later use of loaded data counts the vector memory operations
// issued in between, and a branch that may skip the stores makes it assume
// none were, so it waits for loads issued after the ones it needs.
__device__ __forceinline__ void buf_store8(bf16x4 t, __amdgpu_buffer_rsrc_t r, unsigned off) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, t), r, off, 0, 0);
}

// Four bf16 of one column from four consecutive rows: in each 16-lane group,
// lane i receives element i % 4 of the 8-byte loads of lanes 4e + i / 4, so
// when lane s of the group loads row kb + s / 4, columns nb + 4 (s % 4) .. +3,
// lane i receives rows kb .. kb+3 of column nb + i.
__device__ __forceinline__ bf16x4 tr4(const bf16 *p) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p);
  return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
  return (bf16x8){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Eight bytes of an LDS tile at element offset `off`. The offset is hidden
// from the compiler so that neighbouring reads of the same row are not fused
// into one two-address read (ds_read2_b64): for 16 rows at one column
// offset, that form conflicts many times more on gfx950 LDS than two plain
// 8-byte reads.
__device__ __forceinline__ bf16x4 lds8_apart(const bf16 *tile, int off) {
  asm("" : "+v"(off));
  return *reinterpret_cast<const bf16x4 *>(tile + off);
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ReLU of eight bf16 packed in 16 bytes: every element whose sign bit is set
// becomes +0 (per 32-bit word, m | (m - (m >> 15)) widens each set sign bit
// to a 16-bit mask of its own half; no borrow crosses the halves).
__device__ __forceinline__ u32x4 relu_bf16x8(u32x4 x) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    unsigned m = x[e] & 0x80008000u;
    m |= m - (m >> 15);
    x[e] &= ~m;
  }
  return x;
}

__device__ __forceinline__ bf16x8 ones_bf16x8() {
  const bf16 one = (bf16)1.0f;
  return (bf16x8){one, one, one, one, one, one, one, one};
}

template <int DVT, int DKT = 96>
struct MfCfg {
  static constexpr int C = 64, DK = DKT;
  // LDS row strides (elements). A stride of 8 mod 16 dwords (112 bf16 for 96
  // columns, 80 for 64) keeps both the 16-byte fragment reads (16 rows, one
  // column block) and the transpose reads (rows 4g + l16/4) free of bank
  // conflicts on gfx950 (measured with the LDS conflict counters).
  static constexpr int QS = DK + 16;     // q, k, ks and S^T
  static constexpr int VS = DVT + 16;    // v and the staged output tile
  static constexpr int NCT = DVT / 16;   // 16-column tiles of the dv tile
  static constexpr int NDT = DK / 16;    // 16-row tiles of dk
  static constexpr int NKS = DK / 32;    // 32-deep steps over dk
  static constexpr int NJS = C / 32;     // 32-deep steps over the chunk
  static constexpr int SDT = NDT / 2, SCT = NCT / 2;  // state tiles per state wave
  static constexpr int NQV = DK / 8, NVV = DVT / 8;   // 16-byte vectors per row
  // the published bf16 state: DVT rows of S^T, then (normalised linear
  // attention) one row holding z, read by all lanes as a broadcast
  static constexpr int SROWS = DVT + 1;
  static constexpr int QV = C * NQV / 256;  // q (or k) vectors per role thread
  static constexpr int VV = C * NVV / 256;  // v vectors per state thread
  static constexpr int OV = 16 * NVV / 64;  // output vectors per output lane
  static_assert(C * NQV % 256 == 0 && C * NVV % 256 == 0 && 16 * NVV % 64 == 0, "split");
  static_assert(NCT % 2 == 0 && NDT % 2 == 0, "state split");
};

// Valid rows of chunk ch of an item (0 for chunks past its end).
__device__ __forceinline__ int chunk_rows(const Item &it, int ch) {
  return max(0, min(64, it.t1 - (it.t0 + ch * 64)));
}

// ---------------------------------------------------------------------------
// State role: 4 waves (role thread rt = 0..255, role wave w = 0..3).
//   FUSED: runs beside the output role (also stores raw k for it and
//          publishes the bf16 state each chunk); otherwise the state-only
//          pass that computes a segment's local end state.
//   NORM:  normalised linear attention: k passes through ReLU on its way to
//          LDS, and the waves owning column tiles 0.. (w even) also carry
//          z = sum of decay-weighted k over the chunk rows, as the MFMA of
//          the Ks^T tile with a B operand of ones (every column of the
//          result holds z); z is published in row DVT of the state buffer.
//          Every dv tile's workgroup computes z; the one at c0 = 0 stores it.
//   niter: (state-only pass) run at least this many chunk steps (the
//          barriers of a walk are 1 + its steps rounded up to even).
//   REV:   (state-only pass) the chunks are taken last to first. The local
//          end state is a plain weighted sum, sum_t lambda^(t1-1-t) k_t^T v_t,
//          so each chunk's decay-scaled k carries the decay of the rows after
//          the chunk as well (pc) and the sum is never rescaled; the walk
//          ends on the item's first rows, where the output pass that follows
//          starts, so those k and v rows are still in the last-level cache.
// ---------------------------------------------------------------------------
template <int DVT, bool FUSED, bool NORM = false, int DKT = 96, bool KSR = false,
          bool REV = false>
__device__ __forceinline__ void state_role(
    const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const float *__restrict__ s0, float *__restrict__ s_final,
    float *__restrict__ slots, const Item &it, int idx, int h, int H, int dv,
    int c0, int final_in_slot, int rt, int w, bf16 *sK, bf16 *sKs, bf16 *sV,
    bf16 *sSt0, bf16 *sSt1, const float *sPow, NormPtrs np = NormPtrs{}, int niter = 0) {
  // sK (FUSED only), sKs and sV hold two chunk buffers each. KSR: no
  // decay-scaled copy of k in LDS (it frees a third q/k-sized tile); the
  // raw k tile (sK when FUSED, else sKs) is scaled as its fragments are
  // read, with the same rounding as the copy
  using M = MfCfg<DVT, DKT>;
  static_assert(!(REV && FUSED), "only the state-only pass walks backward");
  constexpr int C = M::C, DK = M::DK, QS = M::QS, VS = M::VS;
  constexpr int SDT = M::SDT, SCT = M::SCT, QV = M::QV, VV = M::VV;
  const int lane = rt & 63, l16 = lane & 15, g = lane >> 4;
  const int tr_row = l16 >> 2, tr_col = 4 * (l16 & 3);
  const unsigned rowKb = (unsigned)(H * DK * 2), rowVb = (unsigned)(H * dv * 2);
  const int nch = (it.t1 - it.t0 + C - 1) / C;
  const int dt0 = SDT * (w >> 1), ct0 = SCT * (w & 1);
  // rows of chunk ch (0 for chunks before the first or past the last)
  auto rows_of = [&](int ch) { return ch < 0 ? 0 : chunk_rows(it, ch); };

  f32x4 accS[SDT][SCT];
  {
    // incoming state: s0 (or zeros) for a sequence's first item, else the
    // combined state in slot idx-1; a local end state starts from zero
    const float *src = nullptr;
    if (FUSED) {
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
  // the normaliser (NORM, waves with w even): z of d tiles dt0 .. dt0+SDT-1
  const bool zw = NORM && !(w & 1);
  f32x4 accZ[SDT];
#pragma unroll
  for (int a = 0; a < SDT; ++a) accZ[a] = (f32x4){0.f, 0.f, 0.f, 0.f};
  if (zw && FUSED) {
    const float *src = nullptr;
    if (it.flags & kFirstSeg)
      src = np.z0 ? np.z0 + ((long long)it.n * H + h) * DK : nullptr;
    else
      src = np.zslots + ((long long)(idx - 1) * H + h) * DK;
    if (src) {
#pragma unroll
      for (int a = 0; a < SDT; ++a)
#pragma unroll
        for (int r = 0; r < 4; ++r) accZ[a][r] = src[16 * (dt0 + a) + 4 * g + r];
    }
  }

  int rowK[QV], colK[QV], rowV[VV], colV[VV];
#pragma unroll
  for (int m = 0; m < QV; ++m) {
    const int vi = rt + 256 * m;
    rowK[m] = vi / M::NQV;
    colK[m] = vi - rowK[m] * M::NQV;
  }
#pragma unroll
  for (int m = 0; m < VV; ++m) {
    const int vi = rt + 256 * m;
    rowV[m] = vi / M::NVV;
    colV[m] = vi - rowV[m] * M::NVV;
  }
  auto load_kv = [&](int ch, u32x4(&rk)[QV], u32x4(&rv)[VV]) {
    const long long tb = (long long)it.t0 + (long long)(ch < 0 ? 0 : ch) * C;
    const unsigned L = (unsigned)rows_of(ch);
    const __amdgpu_buffer_rsrc_t bk = buf_rsrc(k + (tb * H + h) * DK, L * rowKb);
    const __amdgpu_buffer_rsrc_t bv =
        buf_rsrc(v + tb * H * dv + (long long)h * dv + c0, L * rowVb);
#pragma unroll
    for (int m = 0; m < QV; ++m)
      rk[m] = __builtin_amdgcn_raw_buffer_load_b128(bk, rowK[m] * rowKb + colK[m] * 16, 0, 0);
#pragma unroll
    for (int m = 0; m < VV; ++m)
      rv[m] = __builtin_amdgcn_raw_buffer_load_b128(bv, rowV[m] * rowVb + colV[m] * 16, 0, 0);
  };
  constexpr int KBUF = C * QS, VBUF = C * VS;  // elements per chunk buffer
  // pc: an extra decay factor on the whole chunk (REV; 1 otherwise)
  auto store_kv = [&](int L, int buf, float pc, const u32x4(&rk)[QV],
                      const u32x4(&rv)[VV]) {
    bf16 *dK = sK + buf * KBUF, *dV = sV + buf * VBUF;
    bf16 *dKs = KSR && FUSED ? nullptr : sKs + buf * KBUF;
#pragma unroll
    for (int m = 0; m < QV; ++m) {
      const int r = rowK[m];
      const u32x4 kr = NORM ? relu_bf16x8(rk[m]) : rk[m];
      if (FUSED) *reinterpret_cast<u32x4 *>(dK + r * QS + 8 * colK[m]) = kr;
      if (KSR) {
        if (!FUSED) *reinterpret_cast<u32x4 *>(dKs + r * QS + 8 * colK[m]) = kr;
        continue;
      }
      // decay-scaled copy lambda^(L-1-r) k_r; rows past the end are zero
      const float wgt = r < L ? sPow[max(L - 1 - r, 0)] * pc : 0.f;
      const bf16x8 kv = __builtin_bit_cast(bf16x8, kr);
      bf16x8 ks;
#pragma unroll
      for (int e = 0; e < 8; ++e) ks[e] = (bf16)((float)kv[e] * wgt);
      *reinterpret_cast<bf16x8 *>(dKs + r * QS + 8 * colK[m]) = ks;
    }
#pragma unroll
    for (int m = 0; m < VV; ++m)
      *reinterpret_cast<u32x4 *>(dV + rowV[m] * VS + 8 * colV[m]) = rv[m];
  };
  auto publish = [&](bf16 *dst) {
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
    if (zw && l16 == 0) {
#pragma unroll
      for (int a = 0; a < SDT; ++a) {
        bf16x4 t;
#pragma unroll
        for (int r = 0; r < 4; ++r) t[r] = (bf16)accZ[a][r];
        *reinterpret_cast<bf16x4 *>(dst + DVT * QS + 16 * (dt0 + a) + 4 * g) = t;
      }
    }
  };

  // Chunk ch lives in LDS buffer ch & 1. Per chunk: one barrier, then the
  // loads of chunk ch+2 (REV: ch-2) are issued, the registers holding chunk
  // ch+1 (REV: ch-1) are written to the other buffer, and chunk ch is
  // processed. REV: pc_cur is lambda^(rows of the item after chunk ch).
  constexpr int STEP = REV ? -1 : 1;
  const int ch_first = REV ? nch - 1 : 0;
  float pc_cur = 1.0f;
  u32x4 ka[QV], kb[QV], va[VV], vb[VV];
  load_kv(ch_first, ka, va);
  load_kv(ch_first + STEP, kb, vb);
  __syncthreads();  // sPow ready
  store_kv(rows_of(ch_first), ch_first & 1, 1.0f, ka, va);
  if (FUSED) publish(sSt1);  // S_{-1}: the incoming state

  auto body = [&](int ch, u32x4(&rkn)[QV], u32x4(&rvn)[VV], const u32x4(&rkx)[QV],
                  const u32x4(&rvx)[VV], bf16 *st_pub) {
    const int L = rows_of(ch);
    const int cur = ch & 1;
    __syncthreads();  // chunk ch and S_{ch-1} are in LDS; the chunk before is done
    load_kv(ch + 2 * STEP, rkn, rvn);
    // REV: the chunk before ch is followed by ch's rows as well
    const float pc_next = REV ? pc_cur * sPow[L] : 1.0f;
    store_kv(rows_of(ch + STEP), cur ^ 1, pc_next, rkx, rvx);
    const bf16 *cKs = (KSR && FUSED ? sK : sKs) + cur * KBUF, *cV = sV + cur * VBUF;
    const float lamL = sPow[L];
    // KSR: lambda^(L-1-t) for the rows t of this lane's fragments (P k-set),
    // 0 past the chunk's end
    float wk[M::NJS][8];
    if (KSR) {
#pragma unroll
      for (int s = 0; s < M::NJS; ++s)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t0 = 32 * s + 4 * g + e, t1 = t0 + 16;
          wk[s][e] = t0 < L ? sPow[max(L - 1 - t0, 0)] * pc_cur : 0.f;
          wk[s][4 + e] = t1 < L ? sPow[max(L - 1 - t1, 0)] * pc_cur : 0.f;
        }
    }
    if (!REV) {
#pragma unroll
      for (int a = 0; a < SDT; ++a)
#pragma unroll
        for (int b = 0; b < SCT; ++b) accS[a][b] *= lamL;
      if (zw) {
#pragma unroll
        for (int a = 0; a < SDT; ++a) accZ[a] *= lamL;
      }
    }
#pragma unroll
    for (int s = 0; s < M::NJS; ++s) {
      bf16x8 af[SDT], bfr[SCT];
      const int row = 32 * s + 4 * g + tr_row;
#pragma unroll
      for (int a = 0; a < SDT; ++a) {
        const bf16 *base = cKs + row * QS + 16 * (dt0 + a) + tr_col;
        af[a] = cat8(tr4(base), tr4(base + 16 * QS));
        if (KSR) {
#pragma unroll
          for (int e = 0; e < 8; ++e) af[a][e] = (bf16)((float)af[a][e] * wk[s][e]);
        }
      }
#pragma unroll
      for (int b = 0; b < SCT; ++b) {
        const bf16 *base = cV + row * VS + 16 * (ct0 + b) + tr_col;
        bfr[b] = cat8(tr4(base), tr4(base + 16 * VS));
      }
#pragma unroll
      for (int a = 0; a < SDT; ++a)
#pragma unroll
        for (int b = 0; b < SCT; ++b) accS[a][b] = mfma(af[a], bfr[b], accS[a][b]);
      if (zw) {
        const bf16x8 ones = ones_bf16x8();
#pragma unroll
        for (int a = 0; a < SDT; ++a) accZ[a] = mfma(af[a], ones, accZ[a]);
      }
    }
    if (FUSED) publish(st_pub);  // S_ch for the next chunk's readout
    pc_cur = pc_next;
  };
  // a chunk past the end (REV: before the start) is all zeros and leaves
  // the state as it is, so a walk may run longer than the item (niter:
  // two groups of waves that must pass the same barriers)
  const int nit = niter > nch ? niter : nch;
  for (int p = 0; p < nit; p += 2) {
    body(ch_first + STEP * p, ka, va, kb, vb, sSt0);
    body(ch_first + STEP * (p + 1), kb, vb, ka, va, sSt1);
  }

  float *dst = nullptr;
  if (!FUSED || ((it.flags & kLastSeg) && final_in_slot))
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
  if (zw && l16 == 0 && c0 == 0) {
    float *zdst = nullptr;
    if (!FUSED)
      zdst = np.zslots + ((long long)idx * H + h) * DK;
    else if (it.flags & kLastSeg)
      zdst = np.z_final ? np.z_final + ((long long)it.n * H + h) * DK : nullptr;
    if (zdst) {
#pragma unroll
      for (int a = 0; a < SDT; ++a)
#pragma unroll
        for (int r = 0; r < 4; ++r) zdst[16 * (dt0 + a) + 4 * g + r] = accZ[a][r];
    }
  }
}

}  // namespace gla
