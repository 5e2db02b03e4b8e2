// gla_kernels.hip -- HIP kernels of Simple GLA for gfx950 (MI355X).
//
// The recurrence (Laplace 3B / Trainium2 page, section "GLA mixer"):
//     S_t = lambda_h S_{t-1} + k_t^T v_t,      o_t = scale * q_t S_t
// computed chunkwise (same page, section "Challenge 1"). For a chunk of L
// tokens starting from the carried state S_prev, with in-chunk positions
// i, j = 0..L-1:
//     P_ij  = (q_i . k_j) * lambda^(i-j)   if j <= i, else 0
//     o_i   = scale * ( sum_j P_ij v_j  +  lambda^(i+1) q_i S_prev )
//     S_new = lambda^L S_prev + sum_j lambda^(L-1-j) k_j^T v_j
// which is the token recurrence regrouped exactly. Only the state carry is
// sequential across chunks; for long sequences it is further split into time
// segments whose local end states compose as affine maps
//     S_in(g+1) = lambda^(len g) S_in(g) + U_g
// (a scan over segments; U_g is the segment's end state from a zero start).
//
// Kernels:
//   (the bf16 matrix-core forward, d_k 64, 96 or 128, lives in
//   gla_fwd_mfma.hip; the backward in gla_bwd_*.hip)
//   fwd_valu    any supported shape, fp32 or bf16 inputs, fp32 arithmetic
//               on the vector ALUs (the fp32 path and the fallback).
//   planner     varlen: cuts packed sequences into items on the device.
//   order       varlen: workgroup slots take items longest first (a
//               counting sort over chunk counts).
//   combine     scan of segment end states; rcombine and bicombine the
//               backward's reverse scan of carried gradients and both scans
//               in one launch.
//   final_gather, state_fill   a sequence's final state out of its last
//               segment's slot; S_final = S0 for empty sequences.
//   decode      one token per sequence: streams the fp32 state from HBM once
//               (read-modify-write), float4 per lane, readout reduced in LDS;
//               with a slot table for the state pool.
//   zero_i32    clears the chained scan's flags (a fill kernel, so a graph
//               capture of the call holds no memset node).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gla_device.h"
#include "gla_internal.h"

namespace gla {

// ===========================================================================
// Chunked forward on the vector ALUs (fp32 arithmetic, any supported shape)
// ===========================================================================
// One workgroup per (item, head, 16-column dv tile). Everything in LDS as
// fp32: the q/k/v chunk tiles, the masked score tile and the state tile.
// NORM (normalised linear attention): q and k pass through ReLU on load, the
// normaliser z (dk floats, carried like S with v = 1) gives each row its
// denominator phi(q_i) . z_i + eps, which replaces the scale.
constexpr int kValuDvt = 16;

template <typename Tin>
__device__ __forceinline__ float ld_in(const Tin *p) {
  return (float)(*p);
}

template <typename Tin>
__device__ __forceinline__ void st_out(Tin *p, float x) {
  *p = (Tin)x;
}

// gt (gate != kGateNone): the output gate, o = readout * act(g), g in o's
// layout and dtype.
template <typename Tin, bool STATE_ONLY, bool NORM>
__global__ __launch_bounds__(256) void fwd_valu_kernel(
    const Tin *__restrict__ q, const Tin *__restrict__ k,
    const Tin *__restrict__ v, Tin *__restrict__ o,
    const float *__restrict__ s0, float *__restrict__ s_final,
    float *__restrict__ slots, Plan plan, Decay dec, float scale, int H,
    int dk, int dv, int C, int final_in_slot, NormPtrs np, const Tin *__restrict__ gt,
    int gate) {
  extern __shared__ float vsm[];
  float *sQ = vsm;                      // [C][dk]
  float *sK = sQ + C * dk;              // [C][dk]
  float *sV = sK + C * dk;              // [C][16]
  float *sP = sV + C * kValuDvt;        // [C][C]
  float *sS = sP + C * C;               // [dk][16]
  float *sPow = sS + dk * kValuDvt;     // [C+1] (+3)
  float *sZ = sPow + C + 4;             // [dk]   NORM
  float *sDen = sZ + dk;                // [C]    NORM

  const int ndt = dv / kValuDvt;
  int unit, dtile;
  xcd_unit(plan, ndt, plan.max_items * H, unit, dtile);
  if (unit >= plan.max_items * H) return;
  const int slot = unit / H;
  const int h = unit - slot * H;
  int idx;
  Item it;
  if (!slot_item(plan, slot, idx, it)) return;
  if (STATE_ONLY && (it.flags & kLastSeg)) return;

  const int tid = threadIdx.x;
  const int c0 = dtile * kValuDvt;
  const long long rowK = (long long)H * dk, rowV = (long long)H * dv;
  const float lam = dec.lam[h];
  const int len = it.t1 - it.t0;
  const int nch = (len + C - 1) / C;

  for (int n = tid; n <= C; n += blockDim.x) sPow[n] = pow_f64(lam, n);
  {
    const float *src = nullptr;
    if (!STATE_ONLY) {
      if (it.flags & kFirstSeg)
        src = s0 ? s0 + ((long long)it.n * H + h) * dk * dv : nullptr;
      else
        src = slots + ((long long)(idx - 1) * H + h) * dk * dv;
    }
    for (int e = tid; e < dk * kValuDvt; e += blockDim.x) {
      const int d = e / kValuDvt, c = e - d * kValuDvt;
      sS[e] = src ? src[(long long)d * dv + c0 + c] : 0.f;
    }
  }
  if (NORM) {
    const float *zsrc = nullptr;
    if (!STATE_ONLY) {
      if (it.flags & kFirstSeg)
        zsrc = np.z0 ? np.z0 + ((long long)it.n * H + h) * dk : nullptr;
      else
        zsrc = np.zslots + ((long long)(idx - 1) * H + h) * dk;
    }
    for (int d = tid; d < dk; d += blockDim.x) sZ[d] = zsrc ? zsrc[d] : 0.f;
  }
  __syncthreads();

  for (int ch = 0; ch < nch; ++ch) {
    const int tb = it.t0 + ch * C;
    const int L = min(C, it.t1 - tb);
    for (int e = tid; e < C * dk; e += blockDim.x) {
      const int r = e / dk, d = e - r * dk;
      const bool ok = r < L;
      const long long off = (long long)(tb + r) * rowK + (long long)h * dk + d;
      if (!STATE_ONLY) {
        const float x = ok ? ld_in(q + off) : 0.f;
        sQ[e] = NORM ? fmaxf(x, 0.f) : x;
      }
      const float x = ok ? ld_in(k + off) : 0.f;
      sK[e] = NORM ? fmaxf(x, 0.f) : x;
    }
    for (int e = tid; e < C * kValuDvt; e += blockDim.x) {
      const int r = e / kValuDvt, c = e - r * kValuDvt;
      sV[e] = r < L ? ld_in(v + (long long)(tb + r) * rowV + (long long)h * dv + c0 + c) : 0.f;
    }
    __syncthreads();
    if (!STATE_ONLY) {
      for (int e = tid; e < C * C; e += blockDim.x) {
        const int i = e / C, j = e - i * C;
        float acc = 0.f;
        if (j <= i) {
          for (int d = 0; d < dk; ++d) acc = fmaf(sQ[i * dk + d], sK[j * dk + d], acc);
          acc *= sPow[i - j];
        }
        sP[e] = acc;
      }
      __syncthreads();
      if (NORM) {  // per row: phi(q_i) . z_i + eps, z_i = lambda^(i+1) z_prev + sum_j P_ij
        for (int i = tid; i < C; i += blockDim.x) {
          float inter = 0.f;
          for (int d = 0; d < dk; ++d) inter = fmaf(sQ[i * dk + d], sZ[d], inter);
          float intra = 0.f;
          for (int j = 0; j <= i; ++j) intra += sP[i * C + j];
          sDen[i] = fmaf(sPow[i + 1], inter, intra) + kLinearAttnEps;
        }
        __syncthreads();
      }
      for (int e = tid; e < C * kValuDvt; e += blockDim.x) {
        const int i = e / kValuDvt, c = e - i * kValuDvt;
        if (i < L) {
          float inter = 0.f;
          for (int d = 0; d < dk; ++d) inter = fmaf(sQ[i * dk + d], sS[d * kValuDvt + c], inter);
          float intra = 0.f;
          for (int j = 0; j <= i; ++j) intra = fmaf(sP[i * C + j], sV[j * kValuDvt + c], intra);
          const float num = fmaf(sPow[i + 1], inter, intra);
          const long long oi = (long long)(tb + i) * rowV + (long long)h * dv + c0 + c;
          float y = NORM ? num / sDen[i] : scale * num;
          if (gate != kGateNone) y *= gate_act(ld_in(gt + oi), gate);
          st_out(o + oi, y);
        }
      }
      __syncthreads();
    }
    const float lamL = sPow[L];
    for (int e = tid; e < dk * kValuDvt; e += blockDim.x) {
      const int d = e / kValuDvt, c = e - d * kValuDvt;
      float acc = 0.f;
      for (int j = 0; j < L; ++j) acc = fmaf(sPow[L - 1 - j] * sK[j * dk + d], sV[j * kValuDvt + c], acc);
      sS[e] = fmaf(lamL, sS[e], acc);
    }
    if (NORM) {
      for (int d = tid; d < dk; d += blockDim.x) {
        float acc = 0.f;
        for (int j = 0; j < L; ++j) acc = fmaf(sPow[L - 1 - j], sK[j * dk + d], acc);
        sZ[d] = fmaf(lamL, sZ[d], acc);
      }
    }
    __syncthreads();
  }

  float *dst = nullptr;
  if (STATE_ONLY || ((it.flags & kLastSeg) && final_in_slot))
    dst = slots + ((long long)idx * H + h) * dk * dv;
  else if ((it.flags & kLastSeg) && s_final)
    dst = s_final + ((long long)it.n * H + h) * dk * dv;
  if (dst)
    for (int e = tid; e < dk * kValuDvt; e += blockDim.x) {
      const int d = e / kValuDvt, c = e - d * kValuDvt;
      dst[(long long)d * dv + c0 + c] = sS[e];
    }
  if (NORM && c0 == 0) {  // every dv tile holds the same z; the first stores it
    float *zdst = nullptr;
    if (STATE_ONLY)
      zdst = np.zslots + ((long long)idx * H + h) * dk;
    else if (it.flags & kLastSeg)
      zdst = np.z_final ? np.z_final + ((long long)it.n * H + h) * dk : nullptr;
    if (zdst)
      for (int d = tid; d < dk; d += blockDim.x) zdst[d] = sZ[d];
  }
}

// ===========================================================================
// Varlen planner: cut each packed sequence into items of seg_len tokens
// ===========================================================================
// One workgroup of 1024 threads. Thread t takes a contiguous range of
// sequences, counts their segments, a block scan turns counts into offsets,
// then each thread writes its items. index[0] = item count, index[1+n] =
// first item of sequence n (index[1+N] = count). Items past max_items are
// dropped (only reachable with an invalid cu_seqlens).
__global__ __launch_bounds__(1024) void planner_kernel(Plan p, int32_t *index,
                                                       int4 *items) {
  __shared__ int scan[1024];
  const int tid = threadIdx.x;
  const int N = p.n_seq;
  const int per = (N + 1023) / 1024;
  const int nb = min(N, tid * per), ne = min(N, nb + per);
  auto bounds = [&](int n, int &a, int &b) {
    a = clampi(p.cu[n], 0, p.total_T);
    b = clampi(p.cu[n + 1], a, p.total_T);
  };
  int cnt = 0;
  for (int n = nb; n < ne; ++n) {
    int a, b;
    bounds(n, a, b);
    const int L = b - a;
    cnt += L > 0 ? (L + p.seg_len - 1) / p.seg_len : 1;
  }
  scan[tid] = cnt;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int x = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += x;
    __syncthreads();
  }
  int pos = scan[tid] - cnt;  // exclusive prefix
  for (int n = nb; n < ne; ++n) {
    int a, b;
    bounds(n, a, b);
    const int L = b - a;
    const int ns = L > 0 ? (L + p.seg_len - 1) / p.seg_len : 1;
    index[1 + n] = min(pos, p.max_items);
    for (int gi = 0; gi < ns; ++gi, ++pos) {
      if (pos >= p.max_items) continue;
      const int t0 = a + gi * p.seg_len;
      const int t1 = min(t0 + p.seg_len, b);
      const int fl = (gi == 0 ? kFirstSeg : 0) | (gi == ns - 1 ? kLastSeg : 0);
      items[pos] = make_int4(n, t0, t1, fl);
    }
  }
  if (tid == 1023) {
    index[0] = min(scan[1023], p.max_items);
    index[1 + N] = min(scan[1023], p.max_items);
  }
}

// ===========================================================================
// Dispatch order: the plan's items, longest first
// ===========================================================================
// One workgroup. A counting sort of the items by chunk count (descending,
// counts above kOrderBins - 1 share the last bin): an LDS histogram, an
// exclusive scan of the bins, then each item takes the next position of its
// bin. Items of equal chunk count land in no particular order, which changes
// no result (each item's arithmetic is independent of when it runs); giving
// the long items the first workgroups keeps them off the tail of the launch.
constexpr int kOrderBins = 4096;

__global__ __launch_bounds__(1024) void order_kernel(Plan p, int chunk,
                                                     int32_t *order) {
  __shared__ int bins[kOrderBins];
  __shared__ int part[1024];
  const int tid = threadIdx.x;
  const int cnt = p.mode == kPlanVarlenItems ? min(p.index[0], p.max_items)
                                             : min(p.n_seq, p.max_items);
  auto bin_of = [&](int i) {
    Item it;
    if (!load_item(p, i, it)) return kOrderBins - 1;
    const int c = (it.t1 - it.t0 + chunk - 1) / chunk;
    return kOrderBins - 1 - min(c, kOrderBins - 1);
  };
  for (int b = tid; b < kOrderBins; b += 1024) bins[b] = 0;
  __syncthreads();
  for (int i = tid; i < cnt; i += 1024) atomicAdd(&bins[bin_of(i)], 1);
  __syncthreads();
  constexpr int kPer = kOrderBins / 1024;
  int own[kPer], sum = 0;
  for (int j = 0; j < kPer; ++j) {
    own[j] = bins[tid * kPer + j];
    sum += own[j];
  }
  part[tid] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int x = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += x;
    __syncthreads();
  }
  int pos = part[tid] - sum;
  for (int j = 0; j < kPer; ++j) {
    bins[tid * kPer + j] = pos;
    pos += own[j];
  }
  __syncthreads();
  for (int i = tid; i < cnt; i += 1024) order[atomicAdd(&bins[bin_of(i)], 1)] = i;
}

// ===========================================================================
// Segment combine: S_in(i+1) = lambda^(len i) S_in(i) + U_i, in place
// ===========================================================================
// Slot i holds U_i (local end state of item i) on entry and S_in(i+1) on
// exit. One thread per 4 consecutive state elements of one (sequence, head).
// The scan is a chain of scaled adds, but its inputs are not: the slots are
// read in batches of kScanBatch before any of them is rewritten, so a thread
// has that many loads in flight instead of one per step.
constexpr int kScanBatch = 8;

// S <- a S + U over the items of one (sequence, head), forward (REV false:
// items first .. last-2, S starting from s_in) or backward (REV true: items
// last-1 .. first+1); each item's slot receives the running S.
template <bool REV>
__device__ __forceinline__ void scan_slots(const Plan &p, int first, int last, float lam,
                                           float4 S, float *slots, long long stride,
                                           long long off) {
  const int n_steps = last - first - 1;
  for (int b = 0; b < n_steps; b += kScanBatch) {
    float4 U[kScanBatch];
    float a[kScanBatch];
#pragma unroll
    for (int j = 0; j < kScanBatch; ++j) {
      if (b + j < n_steps) {
        const int i = REV ? last - 1 - (b + j) : first + b + j;
        Item it = {0, 0, 0, 0};  // stays empty (a = 1) only for an invalid plan
        load_item(p, i, it);
        a[j] = pow_f64(lam, it.t1 - it.t0);
        U[j] = *reinterpret_cast<const float4 *>(slots + i * stride + off);
      }
    }
#pragma unroll
    for (int j = 0; j < kScanBatch; ++j) {
      if (b + j < n_steps) {
        const int i = REV ? last - 1 - (b + j) : first + b + j;
        S.x = fmaf(a[j], S.x, U[j].x);
        S.y = fmaf(a[j], S.y, U[j].y);
        S.z = fmaf(a[j], S.z, U[j].z);
        S.w = fmaf(a[j], S.w, U[j].w);
        *reinterpret_cast<float4 *>(slots + i * stride + off) = S;
      }
    }
  }
}

__global__ __launch_bounds__(256) void combine_kernel(
    Plan p, const float *__restrict__ s0, float *__restrict__ slots, Decay dec,
    int H, int dk, int dv) {
  const int per_state = dk * dv;
  const int blocks_per = (per_state / 4 + 255) / 256;
  const int unit = blockIdx.x / blocks_per;
  const int part = blockIdx.x - unit * blocks_per;
  const int n = unit / H, h = unit - (unit / H) * H;
  if (n >= p.n_seq) return;
  const int e = (part * 256 + threadIdx.x) * 4;
  if (e >= per_state) return;
  int first, last;
  seq_items(p, n, first, last);
  if (last - first < 2) return;
  float4 S = make_float4(0.f, 0.f, 0.f, 0.f);
  if (s0) S = *reinterpret_cast<const float4 *>(s0 + ((long long)n * H + h) * per_state + e);
  scan_slots<false>(p, first, last, dec.lam[h], S, slots, (long long)H * per_state,
                    (long long)h * per_state + e);
}

// Reverse combine of carried gradients over a sequence's items: slot i
// holds the local carry U_i on entry and, on exit, the carry flowing out of
// item i into item i-1: C_out(i) = lambda^(len i) C_in(i) + U_i, with
// C_in(last) = dL/dS_final (or 0) and C_in(i) = C_out(i+1). One thread per 4
// consecutive state elements of one (sequence, head).
__global__ __launch_bounds__(256) void rcombine_kernel(
    Plan p, const float *__restrict__ ds_final, float *__restrict__ slots, Decay dec,
    int H, int dk, int dv) {
  const int per_state = dk * dv;
  const int blocks_per = (per_state / 4 + 255) / 256;
  const int unit = blockIdx.x / blocks_per;
  const int part = blockIdx.x - unit * blocks_per;
  const int n = unit / H, h = unit - (unit / H) * H;
  if (n >= p.n_seq) return;
  const int e = (part * 256 + threadIdx.x) * 4;
  if (e >= per_state) return;
  int first, last;
  seq_items(p, n, first, last);
  if (last - first < 2) return;
  float4 S = make_float4(0.f, 0.f, 0.f, 0.f);
  if (ds_final)
    S = *reinterpret_cast<const float4 *>(ds_final + ((long long)n * H + h) * per_state + e);
  scan_slots<true>(p, first, last, dec.lam[h], S, slots, (long long)H * per_state,
                   (long long)h * per_state + e);
}

// Both scans of a segmented backward in one launch: workgroups [0, nb)
// combine the forward states (as combine_kernel), the rest the carried
// gradients in reverse (as rcombine_kernel).
__global__ __launch_bounds__(256) void bicombine_kernel(
    Plan p, const float *__restrict__ s0, float *__restrict__ slots,
    const float *__restrict__ ds_final, float *__restrict__ cslots, Decay dec, int H,
    int dk, int dv, int nb) {
  const bool fwd = (int)blockIdx.x < nb;
  const int b = fwd ? (int)blockIdx.x : (int)blockIdx.x - nb;
  const int per_state = dk * dv;
  const int blocks_per = (per_state / 4 + 255) / 256;
  const int unit = b / blocks_per;
  const int part = b - unit * blocks_per;
  const int n = unit / H, h = unit - (unit / H) * H;
  if (n >= p.n_seq) return;
  const int e = (part * 256 + threadIdx.x) * 4;
  if (e >= per_state) return;
  int first, last;
  seq_items(p, n, first, last);
  if (last - first < 2) return;
  const float *init = fwd ? s0 : ds_final;
  float4 S = make_float4(0.f, 0.f, 0.f, 0.f);
  if (init) S = *reinterpret_cast<const float4 *>(init + ((long long)n * H + h) * per_state + e);
  if (fwd)
    scan_slots<false>(p, first, last, dec.lam[h], S, slots, (long long)H * per_state,
                      (long long)h * per_state + e);
  else
    scan_slots<true>(p, first, last, dec.lam[h], S, cslots, (long long)H * per_state,
                     (long long)h * per_state + e);
}

// s_final[n] <- slot of sequence n's last item (in-place final state with
// segments: the last segment cannot write s_final while the first segment of
// the same sequence may still be reading it as s0).
__global__ __launch_bounds__(256) void final_gather_kernel(
    Plan p, const float *__restrict__ slots, float *__restrict__ s_final, int H,
    int dk, int dv) {
  const int per_state = dk * dv;
  const int blocks_per = (per_state / 4 + 255) / 256;
  const int unit = blockIdx.x / blocks_per;
  const int part = blockIdx.x - unit * blocks_per;
  const int n = unit / H, h = unit - (unit / H) * H;
  if (n >= p.n_seq) return;
  const int e = (part * 256 + threadIdx.x) * 4;
  if (e >= per_state) return;
  int first, last;
  seq_items(p, n, first, last);
  if (last <= first) return;
  const float4 x = *reinterpret_cast<const float4 *>(
      slots + ((long long)(last - 1) * H + h) * per_state + e);
  *reinterpret_cast<float4 *>(s_final + ((long long)n * H + h) * per_state + e) = x;
}

// s_final <- s0 (or zeros) for sequences with no tokens in a fixed batch.
__global__ __launch_bounds__(256) void state_fill_kernel(long long n4,
                                                         const float *__restrict__ s0,
                                                         float *__restrict__ s_final) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
  if (s0) x = reinterpret_cast<const float4 *>(s0)[i];
  reinterpret_cast<float4 *>(s_final)[i] = x;
}

// ===========================================================================
// Decode: one token per sequence, state updated in place
// ===========================================================================
// One workgroup per (sequence, head). Thread t owns 4 consecutive columns
// (cq = t % quads) of RPT consecutive rows (row group t / quads). All RPT
// 16-byte loads of the state are issued before any arithmetic, so each
// thread keeps RPT x 16 bytes in flight; every state byte is read once and
// written once, both with non-temporal hints (the 1.5 GB state of a large
// batch has no reuse within a step). (Issuing them before the token vectors
// are staged measured 8 % slower.)
typedef float f32x4n __attribute__((ext_vector_type(4)));

// With a slot table (state pool), row n reads and writes pool entry
// slots[n]; a slot outside [0, n_slots) marks a padding row, whose output
// is written as zeros and which touches no state.
// NORM (normalised linear attention, lambda = 1 from the host): q and k
// pass through ReLU, the normaliser z [rows][dk] is updated in place beside
// the state, and the output is the readout over phi(q) . z + eps.
// gt (gate != kGateNone): the output gate, o = readout * act(g) with g
// [N, H, dv] in o's dtype.
template <typename Tin, int RPT, bool NORM>
__global__ __launch_bounds__(512) void decode_kernel(
    const Tin *__restrict__ q, const Tin *__restrict__ k,
    const Tin *__restrict__ v, Decay dec, float scale, float *__restrict__ state,
    Tin *__restrict__ o, int H, int dk, int dv, int rpt_rt,
    const int32_t *__restrict__ slots, int n_slots, float *__restrict__ zsum,
    const Tin *__restrict__ gt, int gate) {
  extern __shared__ float dsm[];
  const int quads = dv / 4;
  const int rpt = RPT > 0 ? RPT : rpt_rt;
  const int rg_n = dk / rpt;
  float *sq = dsm;        // [dk]
  float *sk = sq + dk;    // [dk]
  float *sv = sk + dk;    // [dv]
  float *part = sv + dv;  // [rg_n][dv]
  float *zt = part + rg_n * dv;  // [dk] (NORM): phi(q)[r] z_new[r]
  const long long unit = blockIdx.x;
  const int h = (int)(unit % H);
  const int tid = threadIdx.x;
  long long srow = unit;  // state row (sequence * H + head)
  if (slots) {
    const int sl = __builtin_amdgcn_readfirstlane(slots[unit / H]);
    if (sl < 0 || sl >= n_slots) {  // padding row
      for (int c = tid; c < dv; c += blockDim.x) o[unit * dv + c] = (Tin)0.f;
      return;
    }
    srow = (long long)sl * H + h;
  }
  const int cq = tid % quads, rg = tid / quads;
  const bool active = rg < rg_n;
  float *base = state + srow * (long long)dk * dv + 4 * cq;
  const int r0 = rg * rpt;
  for (int e = tid; e < dk; e += blockDim.x) {
    const float qe = (float)q[unit * dk + e], ke = (float)k[unit * dk + e];
    sq[e] = NORM ? fmaxf(qe, 0.f) : qe;
    sk[e] = NORM ? fmaxf(ke, 0.f) : ke;
  }
  for (int e = tid; e < dv; e += blockDim.x) sv[e] = (float)v[unit * dv + e];
  __syncthreads();
  const float lam = dec.lam[h];
  if (NORM) {
    for (int e = tid; e < dk; e += blockDim.x) {
      float *zp = zsum + srow * dk + e;
      const float zn = fmaf(lam, *zp, sk[e]);
      *zp = zn;
      zt[e] = sq[e] * zn;
    }
  }
  f32x4n s[RPT > 0 ? RPT : 1];
  if constexpr (RPT > 0) {
    if (active) {
#pragma unroll
      for (int m = 0; m < RPT; ++m)
        s[m] = __builtin_nontemporal_load(reinterpret_cast<f32x4n *>(base + (long long)(r0 + m) * dv));
    }
  }
  f32x4n acc = {0.f, 0.f, 0.f, 0.f};
  if (active) {
    const f32x4n vq = *reinterpret_cast<const f32x4n *>(sv + 4 * cq);
    auto step = [&](f32x4n x, int r) {
      const float kr = sk[r], qr = sq[r];
      x.x = fmaf(lam, x.x, kr * vq.x);
      x.y = fmaf(lam, x.y, kr * vq.y);
      x.z = fmaf(lam, x.z, kr * vq.z);
      x.w = fmaf(lam, x.w, kr * vq.w);
      __builtin_nontemporal_store(x, reinterpret_cast<f32x4n *>(base + (long long)r * dv));
      acc.x = fmaf(qr, x.x, acc.x);
      acc.y = fmaf(qr, x.y, acc.y);
      acc.z = fmaf(qr, x.z, acc.z);
      acc.w = fmaf(qr, x.w, acc.w);
    };
    if constexpr (RPT > 0) {
#pragma unroll
      for (int m = 0; m < RPT; ++m) step(s[m], r0 + m);
    } else {
      for (int m = 0; m < rpt; ++m)
        step(__builtin_nontemporal_load(reinterpret_cast<f32x4n *>(base + (long long)(r0 + m) * dv)),
             r0 + m);
    }
    *reinterpret_cast<f32x4n *>(part + rg * dv + 4 * cq) = acc;
  }
  __syncthreads();
  float coef = scale;
  if (NORM) {
    float den = 0.f;
    for (int r = 0; r < dk; ++r) den += zt[r];
    coef = 1.0f / (den + kLinearAttnEps);
  }
  for (int c = tid; c < dv; c += blockDim.x) {
    float sum = 0.f;
    for (int r = 0; r < rg_n; ++r) sum += part[r * dv + c];
    float y = coef * sum;
    if (gate != kGateNone) y *= gate_act((float)gt[unit * dv + c], gate);
    o[unit * dv + c] = (Tin)y;
  }
}

// ===========================================================================
// launchers
// ===========================================================================
// The matrix-core path runs 64-token chunks (chunk 0 or 64); an explicit 32
// selects the vector-ALU path for these shapes (the host refuses any other
// chunk). Forward and backward take dk 96, 64 or 128.
bool fast_path_ok(int dt, int dk, int dv, int chunk) {
  return dt == 1 && (dk == 96 || dk == 64 || dk == 128) && (dv % 64 == 0) && chunk != 32;
}

int fast_dv_tile(int dv) { return dv % 96 == 0 ? 96 : 64; }

int fwd_dv_tile(int dk, int dv) { return dk == 64 || dk == 128 ? 64 : fast_dv_tile(dv); }

int generic_chunk(int chunk) { return chunk == 32 ? 32 : 64; }

hipError_t launch_planner(const Plan &p, int32_t *index, int4 *items,
                          hipStream_t s) {
  hipLaunchKernelGGL(planner_kernel, dim3(1), dim3(1024), 0, s, p, index, items);
  return hipGetLastError();
}

hipError_t launch_order(const Plan &p, int chunk, int32_t *order, hipStream_t s) {
  hipLaunchKernelGGL(order_kernel, dim3(1), dim3(1024), 0, s, p, chunk, order);
  return hipGetLastError();
}

template <typename Tin, bool SO, bool NORM>
static void launch_valu_n(const Plan &p, const FwdArgs &a, const Decay &dec,
                          int C, hipStream_t s) {
  const int ndt = a.dv / kValuDvt;
  const unsigned grid = xcd_grid(p.deal, (long long)p.max_items * a.H, ndt);
  const size_t lds = sizeof(float) * ((size_t)2 * C * a.dk + C * kValuDvt +
                                      (size_t)C * C + a.dk * kValuDvt + C + 4 +
                                      a.dk + C);
  if (lds > 65536)  // beyond the default dynamic-LDS limit (gfx950 has 160 KB)
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&fwd_valu_kernel<Tin, SO, NORM>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  const NormPtrs np = {a.z0, a.z_final, a.zslots};
  hipLaunchKernelGGL((fwd_valu_kernel<Tin, SO, NORM>), dim3(grid), dim3(256), lds, s,
                     (const Tin *)a.q, (const Tin *)a.k, (const Tin *)a.v,
                     (Tin *)a.o, a.s0, a.s_final, a.slots, p, dec, a.scale,
                     a.H, a.dk, a.dv, C, a.final_in_slot, np, (const Tin *)a.g,
                     SO || NORM ? kGateNone : a.gate);
}

template <typename Tin, bool SO>
static void launch_valu(const Plan &p, const FwdArgs &a, const Decay &dec,
                        int C, hipStream_t s) {
  if (a.norm) launch_valu_n<Tin, SO, true>(p, a, dec, C, s);
  else launch_valu_n<Tin, SO, false>(p, a, dec, C, s);
}

hipError_t launch_fwd(int dt, bool fast, bool state_only, const Plan &p,
                      const FwdArgs &a, const Decay &dec, int chunk,
                      hipStream_t s) {
  if (fast) {
    launch_fwd_mfma(state_only, fwd_dv_tile(a.dk, a.dv), p, a, dec, s);
  } else {
    const int C = generic_chunk(chunk);
    if (dt == 1) {
      if (state_only) launch_valu<bf16, true>(p, a, dec, C, s);
      else launch_valu<bf16, false>(p, a, dec, C, s);
    } else {
      if (state_only) launch_valu<float, true>(p, a, dec, C, s);
      else launch_valu<float, false>(p, a, dec, C, s);
    }
  }
  return hipGetLastError();
}

hipError_t launch_combine(const Plan &p, const FwdArgs &a, const Decay &dec,
                          hipStream_t s) {
  const int per_state = a.dk * a.dv;
  const int blocks_per = (per_state / 4 + 255) / 256;
  const unsigned grid = (unsigned)((long long)p.n_seq * a.H * blocks_per);
  hipLaunchKernelGGL(combine_kernel, dim3(grid), dim3(256), 0, s, p, a.s0,
                     a.slots, dec, a.H, a.dk, a.dv);
  return hipGetLastError();
}

hipError_t launch_rcombine(const Plan &p, const float *ds_final, float *cslots,
                           const Decay &dec, int H, int dk, int dv, hipStream_t s) {
  const int per_state = dk * dv;
  const int blocks_per = (per_state / 4 + 255) / 256;
  const unsigned grid = (unsigned)((long long)p.n_seq * H * blocks_per);
  hipLaunchKernelGGL(rcombine_kernel, dim3(grid), dim3(256), 0, s, p, ds_final,
                     cslots, dec, H, dk, dv);
  return hipGetLastError();
}

hipError_t launch_bicombine(const Plan &p, const float *s0, float *slots,
                            const float *ds_final, float *cslots, const Decay &dec, int H,
                            int dk, int dv, hipStream_t s) {
  const int per_state = dk * dv;
  const int blocks_per = (per_state / 4 + 255) / 256;
  const int nb = p.n_seq * H * blocks_per;
  hipLaunchKernelGGL(bicombine_kernel, dim3((unsigned)(2 * nb)), dim3(256), 0, s, p, s0,
                     slots, ds_final, cslots, dec, H, dk, dv, nb);
  return hipGetLastError();
}

hipError_t launch_final_gather(const Plan &p, const FwdArgs &a, hipStream_t s) {
  const int per_state = a.dk * a.dv;
  const int blocks_per = (per_state / 4 + 255) / 256;
  const unsigned grid = (unsigned)((long long)p.n_seq * a.H * blocks_per);
  hipLaunchKernelGGL(final_gather_kernel, dim3(grid), dim3(256), 0, s, p,
                     a.slots, a.s_final, a.H, a.dk, a.dv);
  return hipGetLastError();
}

// Zeroes n ints (the chained scan's flags): a kernel, not a memset, so that
// a captured graph replays it like any other node.
__global__ __launch_bounds__(256) void zero_i32_kernel(int32_t *__restrict__ p, long long n) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

hipError_t launch_zero_i32(int32_t *p, long long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_i32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_state_fill(int n_states, int H, int dk, int dv,
                             const float *s0, float *s_final, hipStream_t s) {
  const long long n4 = (long long)n_states * H * dk * dv / 4;
  const unsigned grid = (unsigned)((n4 + 255) / 256);
  hipLaunchKernelGGL(state_fill_kernel, dim3(grid), dim3(256), 0, s, n4, s0, s_final);
  return hipGetLastError();
}

hipError_t launch_decode(int dt, int N, int H, int dk, int dv, const void *q,
                         const void *k, const void *v, const Decay &dec,
                         float scale, float *state, void *o, hipStream_t s,
                         const int32_t *slots, int n_slots, float *zsum, const void *g,
                         int gate) {
  const int quads = dv / 4;
  // row groups: the largest divisor of dk with quads * groups <= 320 threads
  // (for dk 96, dv 192: 6 groups of 16 rows, 288 threads)
  int rg = 1;
  for (int c = 1; c <= dk; ++c)
    if (dk % c == 0 && quads * c <= 320) rg = c;
  const int rpt = dk / rg;
  const unsigned threads = (unsigned)(quads * rg);
  const size_t lds = sizeof(float) * (size_t)(2 * dk + dv + rg * dv + (zsum ? dk : 0));
  const unsigned grid = (unsigned)((long long)N * H);
#define GLA_DECODE(T, R, NORM)                                                       \
  hipLaunchKernelGGL((decode_kernel<T, R, NORM>), dim3(grid), dim3(threads), lds, s, \
                     (const T *)q, (const T *)k, (const T *)v, dec, scale,           \
                     state, (T *)o, H, dk, dv, rpt, slots, n_slots, zsum, (const T *)g, gate)
  if (zsum) {
    if (dt == 1) {
      if (rpt == 16) GLA_DECODE(bf16, 16, true);
      else GLA_DECODE(bf16, 0, true);
    } else {
      if (rpt == 16) GLA_DECODE(float, 16, true);
      else GLA_DECODE(float, 0, true);
    }
  } else if (dt == 1) {
    if (rpt == 16) GLA_DECODE(bf16, 16, false);
    else GLA_DECODE(bf16, 0, false);
  } else {
    if (rpt == 16) GLA_DECODE(float, 16, false);
    else GLA_DECODE(float, 0, false);
  }
#undef GLA_DECODE
  return hipGetLastError();
}

}  // namespace gla
