// gla_device.h -- device-side helpers shared by the HIP kernels: vector
// types, fp64 decay powers, the work-item decoding of a Plan and the
// XCD-aware workgroup mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gla_internal.h"

namespace gla {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------
// lambda^n by binary exponentiation in fp64, rounded once to fp32.
__device__ __forceinline__ float pow_f64(float lam, long long n) {
  double r = 1.0, x = (double)lam;
  while (n > 0) {
    if (n & 1) r *= x;
    x *= x;
    n >>= 1;
  }
  return (float)r;
}

// The output gate's activation: sigmoid(z) = 1 / (1 + e^-z), or SiLU(z) =
// z sigmoid(z), with the hardware exponential and reciprocal (about 1e-6
// relative, far below the bf16 rounding of the outputs and the fp32 path's
// tolerance); e^-z overflowing to infinity gives 0, not NaN.
__device__ __forceinline__ float gate_act(float z, int gate) {
  const float s = __builtin_amdgcn_rcpf(1.0f + __expf(-z));
  return gate == kGateSilu ? z * s : s;
}

__host__ __device__ __forceinline__ int clampi(int x, int lo, int hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}

struct Item {
  int n, t0, t1, flags;
};

// Item `idx` of the plan; false when idx is past the last item. (Host and
// device: the host-side plan checks decode items with the same code.)
__host__ __device__ __forceinline__ bool load_item(const Plan &p, int idx, Item &it) {
  if (p.mode == kPlanFixed) {
    if (idx >= p.max_items) return false;
    const int n = idx / p.G;
    const int g = idx - n * p.G;
    const int base = n * p.T;
    it.n = n;
    it.t0 = base + g * p.seg_len;
    it.t1 = min(it.t0 + p.seg_len, base + p.T);
    it.flags = (g == 0 ? kFirstSeg : 0) | (g == p.G - 1 ? kLastSeg : 0);
    return true;
  }
  if (p.mode == kPlanVarlenDirect) {
    if (idx >= p.n_seq) return false;
    const int a = clampi(p.cu[idx], 0, p.total_T);
    const int b = clampi(p.cu[idx + 1], a, p.total_T);
    it.n = idx;
    it.t0 = a;
    it.t1 = b;
    it.flags = kFirstSeg | kLastSeg;
    return true;
  }
  const int cnt = min(p.index[0], p.max_items);
  if (idx >= cnt) return false;
  const int4 x = p.items[idx];
  it.n = x.x;
  it.t0 = x.y;
  it.t1 = x.z;
  it.flags = x.w;
  return true;
}

// Sequence n's item range [first, last) in the plan.
__host__ __device__ __forceinline__ void seq_items(const Plan &p, int n, int &first,
                                          int &last) {
  if (p.mode == kPlanFixed) {
    first = n * p.G;
    last = first + p.G;
  } else if (p.mode == kPlanVarlenDirect) {
    first = n;
    last = n + 1;
  } else {
    const int cap = p.max_items;
    first = clampi(p.index[1 + n], 0, cap);
    last = clampi(p.index[2 + n], first, cap);
  }
}

// Dispatch slot -> (item index, item). Slots are taken longest item first
// when the plan carries an order; false past the last item.
__host__ __device__ __forceinline__ bool slot_item(const Plan &p, int slot, int &idx,
                                          Item &it) {
  int cnt = p.max_items;
  if (p.mode == kPlanVarlenDirect) cnt = p.n_seq;
  else if (p.mode == kPlanVarlenItems) cnt = min(p.index[0], p.max_items);
  if (slot >= cnt) return false;
  idx = p.order ? clampi(p.order[slot], 0, cnt - 1) : slot;
  return load_item(p, idx, it);
}

// The item is the same for every lane of the workgroup; saying so (values
// read back through readfirstlane) lets the compiler keep everything derived
// from it in scalar registers: buffer descriptors built from a value it must
// treat as per-lane cost a loop around every buffer access.
__device__ __forceinline__ void make_uniform(int &idx, Item &it) {
  idx = __builtin_amdgcn_readfirstlane(idx);
  it.n = __builtin_amdgcn_readfirstlane(it.n);
  it.t0 = __builtin_amdgcn_readfirstlane(it.t0);
  it.t1 = __builtin_amdgcn_readfirstlane(it.t1);
  it.flags = __builtin_amdgcn_readfirstlane(it.flags);
}

// Workgroup -> (unit, dv tile). Workgroups are dealt to the 8 XCDs
// round-robin by id (id P runs on XCD P % 8); a unit's dv tiles stay on one
// XCD, so the q and k rows they share are fetched into one L2.
//  - blocked (p.deal == 0): XCD x takes the x-th contiguous eighth of the
//    units, so each XCD streams its own contiguous part of the arrays. Used
//    when every unit carries the same work.
//  - pairs (p.deal == 1): units are taken in pairs (two neighbouring heads of
//    one item, whose q and k rows share a 128-byte line) and the pairs are
//    dealt round-robin over the XCDs, so every XCD gets an equal share of
//    every item. Used when units differ in length (packed sequences, a state
//    pass that skips last segments).
// (xcd_unit_at takes the workgroup id P explicitly: a launch that runs two
// kind of work gives each its own id range starting at a multiple of 8.)
__host__ __device__ __forceinline__ void xcd_unit_at(const Plan &p, int P, int ndt, int units,
                                            int &unit, int &dtile) {
  const int xcd = P & 7;
  const int r = P >> 3;
  if (p.deal == 0) {
    const int per = (units + 7) / 8;
    const int ur = r / ndt;
    unit = xcd * per + ur;
    dtile = r - ur * ndt;
  } else {
    const int per_pair = 2 * ndt;
    const int pr = r / per_pair;
    const int rem = r - pr * per_pair;
    unit = (pr * 8 + xcd) * 2 + rem / ndt;
    dtile = rem - (rem / ndt) * ndt;
  }
}

// The chained scan's workgroups run item-major: id = item * U + u with U =
// H * ndt (a multiple of 8). Within an item, XCD x (= u mod 8) takes the
// x-th eighth of the (head, d_v tile) units in head-major order, so a
// head's d_v tiles (H a multiple of 8 makes U / 8 a multiple of ndt) and
// neighbouring heads share one L2.
__host__ __device__ __forceinline__ void chain_unit(int u, int U, int ndt, int &h, int &dtile) {
  const int su = (u & 7) * (U >> 3) + (u >> 3);
  h = su / ndt;
  dtile = su - h * ndt;
}

__device__ __forceinline__ void xcd_unit(const Plan &p, int ndt, int units,
                                         int &unit, int &dtile) {
  xcd_unit_at(p, (int)blockIdx.x, ndt, units, unit, dtile);
}

// Workgroups xcd_unit needs to cover `units` units of `ndt` dv tiles.
inline unsigned xcd_grid(int deal, long long units, int ndt) {
  if (deal == 0) return (unsigned)((units + 7) / 8 * 8 * ndt);
  const long long pairs = (units + 1) / 2;
  return (unsigned)((pairs + 7) / 8 * 8 * 2 * ndt);
}

}  // namespace gla
