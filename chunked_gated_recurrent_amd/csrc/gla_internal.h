// gla_internal.h -- types shared by the host dispatch (gla_api.cpp) and the
// HIP kernels (gla_*.hip), and the launchers the dispatch calls. Not part of
// the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gla {

constexpr int kMaxHeads = 64;

// Per-head decays, passed to kernels by value (256 bytes of kernel args).
struct Decay {
  float lam[kMaxHeads];
};

// How the token stream is cut into work items. An item is a contiguous token
// range [t0, t1) of one sequence (a whole sequence, or one time segment of a
// long one). Items of one sequence are consecutive; item i > first reads its
// incoming state from slot i-1 of the workspace.
enum PlanMode : int {
  kPlanFixed = 0,         // B sequences of T tokens, G segments each (arithmetic)
  kPlanVarlenDirect = 1,  // one item per packed sequence, bounds from cu_seqlens
  kPlanVarlenItems = 2,   // items written to the workspace by the planner kernel
};

struct Plan {
  int mode;
  int n_seq;      // B or N
  int T;          // fixed mode: tokens per sequence
  int total_T;    // tokens in the packed arrays (bounds clamp)
  int seg_len;    // tokens per segment (a multiple of the chunk)
  int G;          // fixed mode: segments per sequence
  int max_items;  // item slots covered by the launch grids
  const int32_t *cu;     // varlen: [n_seq + 1] device
  const int4 *items;     // kPlanVarlenItems: [max_items] {n, t0, t1, flags}
  const int32_t *index;  // kPlanVarlenItems: [0] = item count, [1 + n] = first item of n
  const int32_t *order;  // optional: dispatch slot -> item, longest item first
  int deal;              // workgroup -> XCD mapping: 0 blocked, 1 pairs round-robin
};

// Item flags
constexpr int kFirstSeg = 1;
constexpr int kLastSeg = 2;

struct FwdArgs {
  const void *q, *k, *v;
  void *o;
  const float *s0;
  float *s_final;
  float *slots;  // [max_items][H][dk][dv] fp32 or nullptr
  float scale;
  int H, dk, dv;
  int final_in_slot;  // last segment writes its final state to its own slot
  // Normalised linear attention (norm = 1): phi = ReLU on q and k, a
  // normaliser sum z carried beside S, o = phi(q) S / (phi(q) . z + eps)
  int norm;
  const float *z0;  // [n_seq][H][dk] or nullptr
  float *z_final;   // [n_seq][H][dk] or nullptr
  float *zslots;    // [max_items][H][dk] with time segments
  // output gate (gate != kGateNone): g has o's layout and dtype
  const void *g;
  int gate;
};

constexpr float kLinearAttnEps = 1e-6f;

// Output gate applied to the mixer's output, y = o * act(g): none, sigmoid
// or SiLU (the values of the public gla_gate enum).
constexpr int kGateNone = 0, kGateSigmoid = 1, kGateSilu = 2;

// Normalised linear attention: where the normaliser sum z enters and leaves
// (all [.][H][dk] fp32, nullptr when absent); kernel argument.
struct NormPtrs {
  const float *z0;  // incoming z of each sequence
  float *z_final;   // z after each sequence's last token
  float *zslots;    // per-item z of time segments (local end, then combined)
};

struct BwdArgs {
  const void *q, *k, *v, *dout;
  const float *s0, *ds_final;
  void *dq, *dk, *dv_out;
  float *ds0;
  float *slots;              // time segments: incoming states (forward combine)
  float *cslots;             // time segments: carried gradients (reverse combine)
  float *part_dq, *part_dk;  // [dv tiles][H][tokens][96] fp32 partial sums
  float scale;
  int H, dv;
  int dk_dim;  // dk
};

// ---- launchers (gla_kernels.hip) -------------------------------------------
// All return the hipGetLastError() of their launches.
bool fast_path_ok(int dt, int dk, int dv, int chunk);
int fast_dv_tile(int dv);
int fwd_dv_tile(int dk, int dv);
int generic_chunk(int chunk);
hipError_t launch_planner(const Plan &p, int32_t *index, int4 *items, hipStream_t s);
hipError_t launch_order(const Plan &p, int chunk, int32_t *order, hipStream_t s);

// Plans with more items than this run in index order (no dispatch order).
constexpr int kOrderMaxItems = 16384;
hipError_t launch_fwd(int dt, bool fast, bool state_only, const Plan &p,
                      const FwdArgs &a, const Decay &dec, int chunk,
                      hipStream_t s);
hipError_t launch_short_conv_fwd(int dt, int B, int T, int D, const void *x,
                                 const float *w, const float *bias, const float *win_in,
                                 void *y, float *win_out, hipStream_t s);
hipError_t launch_short_conv_decode(int dt, int N, int D, const void *x, const float *w,
                                    const float *bias, float *window, void *y,
                                    hipStream_t s);
hipError_t launch_rcombine(const Plan &p, const float *ds_final, float *cslots,
                           const Decay &dec, int H, int dk, int dv, hipStream_t s);
hipError_t launch_bwd_mfma(int dvt, const Plan &p, const BwdArgs &a,
                           const Decay &dec, hipStream_t s);
// time segments of the matrix-core backward: the forward's local end states
// (slots) and the local carries (cslots) in one launch, then both scans
hipError_t launch_bwd_boundary(int dvt, const Plan &p, const BwdArgs &a,
                               const Decay &dec, hipStream_t s);
hipError_t launch_bicombine(const Plan &p, const float *s0, float *slots,
                            const float *ds_final, float *cslots, const Decay &dec, int H,
                            int dk, int dv, hipStream_t s);
// matrix-core backward with one workgroup per (item, head) over all of dv
// (gla_bwd_wide.hip), no partial sums. pair: two time segments per sequence
// joined on load; fused: no time segments, both walks in one launch, with
// the dk and dv rows of the last tail_q16 / 65536 of every sequence's
// chunks formed by its dq walk's workgroup
bool bwd_wide_ok(int dk, int dv);
hipError_t launch_bwd_wide(const Plan &p, const BwdArgs &a, const Decay &dec, int pair,
                           bool fused, int tail_q16, hipStream_t s);
// vector-ALU backward (gla_bwd_valu.hip): dv tiles of valu_bwd_tile(dv)
// columns, fp32 partial rows [dv tile][H][token][dk]
int valu_bwd_tile(int dv);
hipError_t launch_bwd_valu(int dt, const Plan &p, const BwdArgs &a, const Decay &dec,
                           hipStream_t s);
void launch_fwd_mfma(bool state_only, int dvt, const Plan &p, const FwdArgs &a,
                     const Decay &dec, hipStream_t s);
hipError_t launch_combine(const Plan &p, const FwdArgs &a, const Decay &dec,
                          hipStream_t s);
// Segmented bf16 forward (matrix cores, no normaliser) in one launch, the
// chained scan (gla_fwd_mfma.hip): a.slots, incl and sin each
// [max_items][H][dk][dv] fp32 (local, inclusive and incoming states), flags
// [max_items][H][dv / dvt] ints, zeroed before the launch.
bool fwd_chain_ok(int dk, int H, int items_per_seq);
void launch_fwd_chain(int dvt, const Plan &p, const FwdArgs &a, const Decay &dec, float *incl,
                      float *sin, int *flags, hipStream_t s);
hipError_t launch_zero_i32(int32_t *p, long long n, hipStream_t s);
hipError_t launch_final_gather(const Plan &p, const FwdArgs &a, hipStream_t s);
hipError_t launch_state_fill(int n_states, int H, int dk, int dv,
                             const float *s0, float *s_final, hipStream_t s);
hipError_t launch_decode(int dt, int N, int H, int dk, int dv, const void *q,
                         const void *k, const void *v, const Decay &dec,
                         float scale, float *state, void *o, hipStream_t s,
                         const int32_t *slots = nullptr, int n_slots = 0,
                         float *zsum = nullptr, const void *g = nullptr,
                         int gate = kGateNone);

}  // namespace gla
