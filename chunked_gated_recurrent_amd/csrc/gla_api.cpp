// gla_api.cpp -- the C ABI declared in include/gla.h: host-side validation,
// work planning and kernel dispatch. Validation and planning make no HIP
// call, so every error path is testable on a machine without a GPU.
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "gla.h"
#include "gla_internal.h"

using namespace gla;

// Debug builds (-DGLA_DEBUG; the host sanitizer tests build one) check the
// plan and workspace arithmetic as it is made; release builds compile the
// checks away.
#ifdef GLA_DEBUG
#include <stdio.h>
#define GLA_HOST_CHECK(c)                                                       \
  do {                                                                          \
    if (!(c)) {                                                                 \
      fprintf(stderr, "%s:%d: plan check failed: %s\n", __FILE__, __LINE__, #c); \
      abort();                                                                  \
    }                                                                           \
  } while (0)
#else
#define GLA_HOST_CHECK(c) ((void)0)
#endif

namespace {

constexpr long long kMaxTokens = 0x7fffffffLL;  // token indices are int32 on device

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

gla_status check_common(int dt, int H, int dk, int dv, int chunk) {
  if (dt != GLA_F32 && dt != GLA_BF16) return GLA_ERR_DTYPE;
  if (H < 1 || dk < 1 || dv < 1) return GLA_ERR_SHAPE;
  if (H > GLA_MAX_HEADS) return GLA_ERR_UNSUPPORTED;
  if (dk % 16 != 0 || dv % 16 != 0 || dk > 128 || dv > 256) return GLA_ERR_UNSUPPORTED;
  // 0 (the library default, 64), 32 (vector ALUs) or 64; no kernel runs
  // 128-token chunks, so 128 is refused rather than served with 64
  if (chunk != 0 && chunk != 32 && chunk != 64) return GLA_ERR_UNSUPPORTED;
  return GLA_OK;
}

gla_status check_decay(const float *d, int H) {
  if (!d) return GLA_ERR_NULL;
  for (int h = 0; h < H; ++h) {
    const float x = d[h];
    if (!isfinite(x) || !(x > 0.0f) || x > 1.0f) return GLA_ERR_DECAY;
  }
  return GLA_OK;
}

bool misaligned(const void *p) { return p && ((uintptr_t)p & 15u) != 0; }

// The public gate codes map one to one onto the kernels' (checked below);
// anything else, "no gate" included, becomes a code check_gate refuses.
int gate_code(gla_gate g) {
  return (g == GLA_GATE_SIGMOID || g == GLA_GATE_SILU) ? (int)g : -1;
}

gla_status check_gate(int gate) {
  static_assert(GLA_GATE_SIGMOID == kGateSigmoid && GLA_GATE_SILU == kGateSilu, "gate codes");
  if (gate != kGateNone && gate != kGateSigmoid && gate != kGateSilu) return GLA_ERR_UNSUPPORTED;
  return GLA_OK;
}

// [a, a+na) and [b, b+nb) share a byte (empty ranges never overlap)
bool overlap(const void *a, size_t na, const void *b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// Workgroups a call should have in flight before it pays for splitting
// sequences into time segments (one per compute unit on a 256-CU part: the
// matrix-core kernels hold one workgroup per CU).
int target_workgroups() {
  const char *e = getenv("GLA_TARGET_WGS");
  if (e && *e) {
    const long v = strtol(e, nullptr, 10);
    if (v >= 1 && v <= (1L << 20)) return (int)v;
  }
  return 256;
}

// Share of every sequence's chunks (in 1/65536) whose dk and dv rows the
// fused backward gives to the dq walk's workgroup when both walks fit one
// round of the CUs. A chunk of the reverse walk costs about 1.45 times one
// of the dq walk, and the reverse workgroup still carries the gradient
// through the chunks it gives away, so the split that evens out the two
// was measured per d_k (B8 T2048 H16, us per call at shares 1/4 and 3/16):
// d_k 64 at 1/4 (d_v 192: 154 against 162), d_k 96 and 128 at 3/16 (d_k
// 96, d_v 192: 179 against 184; d_k 128, d_v 128: 167 against 176).
// GLA_BWD_TAIL (a fraction in [0, 0.5]) overrides it.
int bwd_tail_q16(int dk) {
  const char *e = getenv("GLA_BWD_TAIL");
  if (e && *e) {
    const double f = strtod(e, nullptr);
    if (f >= 0.0 && f <= 0.5) return (int)(f * 65536.0 + 0.5);
  }
  return dk <= 64 ? 16384 : 12288;
}

struct HostPlan {
  Plan p;
  bool fast;
  int chunk;      // tokens per chunk the kernels use
  int ndt;        // dv tiles per (item, head)
  bool segmented; // at least one sequence has more than one item
  bool ordered;   // items are dispatched longest first (order in workspace)
  bool chain;     // time segments in one launch (the chained scan)
  size_t off_index, off_items, off_order, off_slots, ws_bytes;
  size_t off_incl, off_sin, off_flags;  // chained scan: inclusive and incoming states, flags
  size_t off_zslots;  // normalised linear attention with time segments
};

void base_plan(HostPlan &hp, int dt, int dk, int dv, int chunk) {
  memset(&hp, 0, sizeof(hp));
  hp.fast = fast_path_ok(dt, dk, dv, chunk);
  hp.chunk = hp.fast ? 64 : generic_chunk(chunk);
  hp.ndt = hp.fast ? dv / fwd_dv_tile(dk, dv) : dv / 16;
}

// plan_ndt (when > 0) replaces the forward's dv tiles per unit in the
// decision to split sequences into time segments (the wide backward runs
// one workgroup per unit).
HostPlan plan_fixed(int dt, int B, int T, int H, int dk, int dv, int chunk,
                    int plan_ndt = 0) {
  HostPlan hp;
  base_plan(hp, dt, dk, dv, chunk);
  const int C = hp.chunk;
  const long long chains = (long long)B * H * (plan_ndt > 0 ? plan_ndt : hp.ndt);
  const long long target = target_workgroups();
  int G = 1;
  if (T > 2 * C && chains < target) {
    const long long want = (target + chains - 1) / chains;
    const long long maxg = (T + 2 * C - 1) / (2 * C);  // segments of >= 2 chunks
    G = (int)(want < maxg ? want : maxg);
    if (G < 1) G = 1;
  }
  int seg = T > 0 ? (T + G - 1) / G : C;
  seg = ((seg + C - 1) / C) * C;
  G = T > 0 ? (T + seg - 1) / seg : 1;
  Plan &p = hp.p;
  p.mode = kPlanFixed;
  p.n_seq = B;
  p.T = T;
  p.total_T = (int)((long long)B * T);
  p.seg_len = seg;
  p.G = G;
  p.max_items = B * G;
  hp.segmented = G > 1;
  hp.off_slots = 0;
  hp.ws_bytes = hp.segmented ? (size_t)B * G * H * dk * dv * sizeof(float) : 0;
  // segments are whole chunks, cover the sequence, and none is empty
  GLA_HOST_CHECK(C > 0 && seg > 0 && seg % C == 0 && G >= 1);
  GLA_HOST_CHECK((long long)seg * G >= T);
  GLA_HOST_CHECK(T == 0 || (long long)seg * (G - 1) < T);
  GLA_HOST_CHECK((long long)p.max_items == (long long)B * G);
  return hp;
}

HostPlan plan_varlen(int dt, int N, int total_T, int H, int dk, int dv, int chunk,
                     int plan_ndt = 0) {
  HostPlan hp;
  base_plan(hp, dt, dk, dv, chunk);
  const int C = hp.chunk;
  const long long chains = (long long)N * H * (plan_ndt > 0 ? plan_ndt : hp.ndt);
  const long long target = target_workgroups();
  Plan &p = hp.p;
  p.n_seq = N;
  p.total_T = total_T;
  const long long avg = N > 0 ? (long long)total_T / N : 0;
  if (chains >= target || avg <= 2 * C) {
    p.mode = kPlanVarlenDirect;
    p.max_items = N;
    p.seg_len = total_T > 0 ? total_T : C;
    p.G = 1;
    hp.segmented = false;
    hp.ordered = N > 1 && N <= kOrderMaxItems;
    hp.off_order = 0;
    hp.ws_bytes = hp.ordered ? align256(sizeof(int32_t) * (size_t)N) : 0;
    GLA_HOST_CHECK(!hp.ordered || hp.ws_bytes >= sizeof(int32_t) * (size_t)N);
    return hp;
  }
  const long long want = (target + chains - 1) / chains;  // segments per sequence
  long long seg = (avg + want - 1) / want;
  if (seg < 2 * C) seg = 2 * C;
  seg = ((seg + C - 1) / C) * C;
  p.mode = kPlanVarlenItems;
  p.seg_len = (int)seg;
  p.G = 0;
  p.max_items = (int)(N + total_T / seg);
  hp.segmented = true;
  hp.ordered = p.max_items <= kOrderMaxItems;
  hp.off_index = 0;
  hp.off_items = align256(sizeof(int32_t) * ((size_t)N + 2));
  hp.off_order = hp.off_items + align256(sizeof(int4) * (size_t)p.max_items);
  hp.off_slots = hp.off_order +
                 (hp.ordered ? align256(sizeof(int32_t) * (size_t)p.max_items) : 0);
  hp.ws_bytes = hp.off_slots + (size_t)p.max_items * H * dk * dv * sizeof(float);
  // a sequence of L tokens becomes ceil(L / seg) items (one if empty), and
  // sum_n ceil(L_n / seg) <= N + total_T / seg: the item slots suffice
  GLA_HOST_CHECK(seg % C == 0 && seg >= 2 * C);
  GLA_HOST_CHECK(p.max_items >= N);
  // index, item table, order and state slots: 256-byte aligned, in this
  // order, without overlap
  GLA_HOST_CHECK(hp.off_index == 0 && hp.off_items % 256 == 0 && hp.off_order % 256 == 0 &&
                 hp.off_slots % 256 == 0);
  GLA_HOST_CHECK(hp.off_items >= sizeof(int32_t) * ((size_t)N + 2));
  GLA_HOST_CHECK(hp.off_order >= hp.off_items + sizeof(int4) * (size_t)p.max_items);
  GLA_HOST_CHECK(hp.off_slots >= hp.off_order +
                                     (hp.ordered ? sizeof(int32_t) * (size_t)p.max_items : 0));
  return hp;
}

// GLA_FWD_CHAIN=1 runs the bf16 forward of a fixed batch with time segments
// in one launch (fwd_chain_kernel: local states, chained combine and
// outputs) instead of three (state pass, combine, output pass). The three
// launches are the default: at one 65,536-token sequence of 16 heads they
// take 369 us per call against 493 us for the chained scan.
bool fwd_chain_enabled() {
  const char *e = getenv("GLA_FWD_CHAIN");
  return e && e[0] == '1' && e[1] == 0;
}

HostPlan plan_fwd_fixed(int dt, int B, int T, int H, int dk, int dv, int chunk) {
  HostPlan hp = plan_fixed(dt, B, T, H, dk, dv, chunk);
  if (hp.fast && hp.segmented && fwd_chain_ok(dk, H, hp.p.G) && fwd_chain_enabled()) {
    const size_t slot_bytes = (size_t)hp.p.max_items * H * dk * dv * sizeof(float);
    const size_t flag_bytes = (size_t)hp.p.max_items * H * hp.ndt * sizeof(int32_t);
    hp.chain = true;
    hp.off_incl = align256(hp.off_slots + slot_bytes);
    hp.off_sin = align256(hp.off_incl + slot_bytes);
    hp.off_flags = align256(hp.off_sin + slot_bytes);
    hp.ws_bytes = hp.off_flags + flag_bytes;
    // local, inclusive and incoming states, then flags: 256-byte aligned, in
    // this order, without overlap
    GLA_HOST_CHECK(hp.off_slots == 0 && hp.off_incl % 256 == 0 && hp.off_sin % 256 == 0 &&
                   hp.off_flags % 256 == 0);
    GLA_HOST_CHECK(hp.off_incl >= slot_bytes && hp.off_sin >= hp.off_incl + slot_bytes &&
                   hp.off_flags >= hp.off_sin + slot_bytes);
  }
  return hp;
}

Decay make_decay(const float *d, int H) {
  Decay dec;
  memset(&dec, 0, sizeof(dec));
  for (int h = 0; h < H; ++h) dec.lam[h] = d[h];
  return dec;
}

// Launch the planned forward: [planner] -> [local end states -> combine] ->
// outputs -> [final gather], or, for the chained scan, [flag reset] ->
// one launch -> [final gather].
gla_status run_forward(int dt, const HostPlan &hp, FwdArgs a, const Decay &dec,
                       void *workspace, hipStream_t s) {
  Plan p = hp.p;
  char *ws = (char *)workspace;
  (void)hipGetLastError();  // report only this call's launch errors
  if (p.mode == kPlanVarlenItems) {
    p.index = (const int32_t *)(ws + hp.off_index);
    p.items = (const int4 *)(ws + hp.off_items);
    if (launch_planner(p, (int32_t *)(ws + hp.off_index), (int4 *)(ws + hp.off_items), s) != hipSuccess)
      return GLA_ERR_HIP;
  }
  if (hp.ordered) {
    if (launch_order(p, hp.chunk, (int32_t *)(ws + hp.off_order), s) != hipSuccess)
      return GLA_ERR_HIP;
    p.order = (const int32_t *)(ws + hp.off_order);
  }
  // Units of a packed batch differ in length: deal them in pairs over the
  // XCDs. A fixed batch's output pass has equal units: blocked.
  p.deal = p.mode == kPlanFixed ? 0 : 1;
  if (hp.chain) {
    a.slots = (float *)(ws + hp.off_slots);
    float *incl = (float *)(ws + hp.off_incl);
    float *sin = (float *)(ws + hp.off_sin);
    int32_t *flags = (int32_t *)(ws + hp.off_flags);
    // in place (s_final == s0): the first items' look-backs read s0, so the
    // last item writes its final state to its own slot of sin and a gather
    // copies it out after the launch
    a.final_in_slot = (a.s_final && a.s_final == a.s0) ? 1 : 0;
    if (launch_zero_i32(flags, (long long)p.max_items * a.H * hp.ndt, s) != hipSuccess)
      return GLA_ERR_HIP;
    launch_fwd_chain(a.dv / hp.ndt, p, a, dec, incl, sin, flags, s);
    if (hipGetLastError() != hipSuccess) return GLA_ERR_HIP;
    if (a.final_in_slot) {
      FwdArgs g = a;
      g.slots = sin;
      if (launch_final_gather(p, g, s) != hipSuccess) return GLA_ERR_HIP;
    }
    return GLA_OK;
  }
  if (hp.segmented) {
    a.slots = (float *)(ws + hp.off_slots);
    if (a.norm) a.zslots = (float *)(ws + hp.off_zslots);
    Plan ps = p;
    ps.deal = 1;  // the state pass skips every last segment
    if (launch_fwd(dt, hp.fast, true, ps, a, dec, hp.chunk, s) != hipSuccess) return GLA_ERR_HIP;
    if (launch_combine(p, a, dec, s) != hipSuccess) return GLA_ERR_HIP;
    if (a.norm) {  // the normaliser composes like a state with one column
      FwdArgs az = a;
      az.s0 = a.z0;
      az.slots = a.zslots;
      az.dv = 1;
      if (launch_combine(p, az, dec, s) != hipSuccess) return GLA_ERR_HIP;
    }
    // In place (s_final == s0): the first segment reads s0 while the last
    // writes the final state, so the last writes its own slot and a gather
    // copies it out afterwards.
    a.final_in_slot = (a.s_final && a.s_final == a.s0) ? 1 : 0;
  }
  if (launch_fwd(dt, hp.fast, false, p, a, dec, hp.chunk, s) != hipSuccess) return GLA_ERR_HIP;
  if (a.final_in_slot && launch_final_gather(p, a, s) != hipSuccess) return GLA_ERR_HIP;
  return GLA_OK;
}

size_t elem_size(int dt) { return dt == GLA_BF16 ? 2 : 4; }

// Normalised linear attention: the forward's plan plus, with time segments,
// one z slot ([item][H][dk] fp32) per item after the state slots.
HostPlan with_zslots(HostPlan hp, int H, int dk) {
  if (hp.segmented) {
    [[maybe_unused]] const size_t state_end = hp.ws_bytes;  // read by the debug checks
    hp.off_zslots = align256(hp.ws_bytes);
    hp.ws_bytes = hp.off_zslots + (size_t)hp.p.max_items * H * dk * sizeof(float);
    GLA_HOST_CHECK(hp.off_zslots % 256 == 0 && hp.off_zslots >= state_end);
  }
  return hp;
}

HostPlan plan_linear_attn(int dt, int B, int T, int H, int dk, int dv, int chunk) {
  return with_zslots(plan_fixed(dt, B, T, H, dk, dv, chunk), H, dk);
}

HostPlan plan_linear_attn_varlen(int dt, int N, int total_T, int H, int dk, int dv,
                                 int chunk) {
  return with_zslots(plan_varlen(dt, N, total_T, H, dk, dv, chunk), H, dk);
}

Decay unit_decay() {
  Decay one;
  for (int h = 0; h < kMaxHeads; ++h) one.lam[h] = 1.0f;
  return one;
}

// Backward layout: the forward's plan (work items, dispatch order, time
// segments and their incoming-state slots, in the forward's workspace
// layout), then, with time segments, the carried-gradient slots, then the
// fp32 dv-tile partials of dq and dk ([dv tile][H][token][dk] each). Dv
// tiles of 96 or 64 columns on the matrix-core path, of up to 64 on the
// vector-ALU path.
// The wide matrix-core backward (dk 96, dv 192: one workgroup per unit over
// all of dv) writes dq and dk directly: no partials.
struct BwdPlan {
  HostPlan hp;
  int ndt, dvt;
  bool wide;
  size_t off_cslots, off_part, part_bytes, ws_bytes;
};

bool bwd_wide_path(int dt, int dk, int dv, int chunk) {
  return fast_path_ok(dt, dk, dv, chunk) && bwd_wide_ok(dk, dv);
}

// dv tiles per unit the backward plans its time segments for
int bwd_plan_ndt(int dt, int dk, int dv, int chunk) {
  if (bwd_wide_path(dt, dk, dv, chunk)) return 1;
  return fast_path_ok(dt, dk, dv, chunk) ? dv / fwd_dv_tile(dk, dv) : 0;
}

// The backward's plan. On the workgroup-per-head path both walks can run in
// one launch when no sequence needs time segments (two workgroups per unit,
// so half the units fill the GPU): plan for that first, and fall back to
// time segments (walks launched one after the other, one workgroup per
// unit) only if it still needs them.
HostPlan bwd_plan_fixed(int dt, int B, int T, int H, int dk, int dv, int chunk) {
  if (bwd_wide_path(dt, dk, dv, chunk)) {
    const HostPlan one = plan_fixed(dt, B, T, H, dk, dv, chunk, 2);
    if (!one.segmented) return one;
  }
  return plan_fixed(dt, B, T, H, dk, dv, chunk, bwd_plan_ndt(dt, dk, dv, chunk));
}

HostPlan bwd_plan_varlen(int dt, int N, int total_T, int H, int dk, int dv, int chunk) {
  if (bwd_wide_path(dt, dk, dv, chunk)) {
    const HostPlan one = plan_varlen(dt, N, total_T, H, dk, dv, chunk, 2);
    if (!one.segmented) return one;
  }
  return plan_varlen(dt, N, total_T, H, dk, dv, chunk, bwd_plan_ndt(dt, dk, dv, chunk));
}

BwdPlan bwd_layout(const HostPlan &hp, long long total_T, int H, int dk, int dv) {
  BwdPlan bp;
  memset(&bp, 0, sizeof(bp));
  bp.hp = hp;
  bp.wide = hp.fast && bwd_wide_ok(dk, dv);
  bp.dvt = bp.wide ? dv : hp.fast ? fwd_dv_tile(dk, dv) : valu_bwd_tile(dv);
  bp.ndt = dv / bp.dvt;
  const size_t base = align256(hp.ws_bytes);
  const size_t slot_bytes =
      hp.segmented ? align256((size_t)hp.p.max_items * H * dk * dv * sizeof(float)) : 0;
  bp.off_cslots = base;
  bp.off_part = base + slot_bytes;
  bp.part_bytes = bp.wide ? 0 : align256((size_t)bp.ndt * H * total_T * dk * sizeof(float));
  bp.ws_bytes = total_T > 0 ? bp.off_part + 2 * bp.part_bytes : 0;
  // the forward's layout, then the carried-gradient slots, then the two
  // partial-sum arrays, each 256-byte aligned and after the one before
  GLA_HOST_CHECK(bp.ndt >= 1 && bp.dvt * bp.ndt == dv);
  GLA_HOST_CHECK(bp.off_cslots % 256 == 0 && bp.off_cslots >= hp.ws_bytes);
  GLA_HOST_CHECK(bp.off_part % 256 == 0 && bp.part_bytes % 256 == 0);
  GLA_HOST_CHECK(!hp.segmented ||
                 bp.off_part >= bp.off_cslots + (size_t)hp.p.max_items * H * dk * dv * 4);
  return bp;
}

// Launch the planned backward: [planner] [order] [forward state pass ->
// combine] -> [carry pass -> reverse combine] -> dq pass -> dk/dv pass ->
// partial sums.
gla_status run_backward(int dt, const BwdPlan &bp, BwdArgs a, const Decay &dec,
                        void *workspace, hipStream_t s) {
  const HostPlan &hp = bp.hp;
  Plan p = hp.p;
  char *ws = (char *)workspace;
  (void)hipGetLastError();  // report only this call's launch errors
  if (p.mode == kPlanVarlenItems) {
    p.index = (const int32_t *)(ws + hp.off_index);
    p.items = (const int4 *)(ws + hp.off_items);
    if (launch_planner(p, (int32_t *)(ws + hp.off_index), (int4 *)(ws + hp.off_items), s) != hipSuccess)
      return GLA_ERR_HIP;
  }
  if (hp.ordered) {
    if (launch_order(p, hp.chunk, (int32_t *)(ws + hp.off_order), s) != hipSuccess)
      return GLA_ERR_HIP;
    p.order = (const int32_t *)(ws + hp.off_order);
  }
  p.deal = p.mode == kPlanFixed ? 0 : 1;
  a.part_dq = (float *)(ws + bp.off_part);
  a.part_dk = (float *)(ws + bp.off_part + bp.part_bytes);
  bool pair = false;
  if (hp.segmented) {
    // the segments' incoming forward states (the forward's state pass and
    // combine) and, on the matrix cores, their incoming carried gradients
    // (local carries and the reverse combine); the vector-ALU backward runs
    // its own carry pass
    a.slots = (float *)(ws + hp.off_slots);
    a.cslots = (float *)(ws + bp.off_cslots);
    if (hp.fast) {
      if (launch_bwd_boundary(fwd_dv_tile(a.dk_dim, a.dv), p, a, dec, s) != hipSuccess)
        return GLA_ERR_HIP;
      // two segments per sequence: the wide kernels join them on load
      pair = bp.wide && p.mode == kPlanFixed && p.G == 2;
      if (!pair && launch_bicombine(p, a.s0, a.slots, a.ds_final, a.cslots, dec, a.H,
                                    a.dk_dim, a.dv, s) != hipSuccess)
        return GLA_ERR_HIP;
    } else {
      FwdArgs f;
      memset(&f, 0, sizeof(f));
      f.q = a.q; f.k = a.k; f.v = a.v; f.s0 = a.s0; f.slots = a.slots;
      f.scale = a.scale; f.H = a.H; f.dk = a.dk_dim; f.dv = a.dv;
      Plan ps = p;
      ps.deal = 1;  // the state pass skips every last segment
      if (launch_fwd(dt, false, true, ps, f, dec, hp.chunk, s) != hipSuccess) return GLA_ERR_HIP;
      if (launch_combine(p, f, dec, s) != hipSuccess) return GLA_ERR_HIP;
    }
  }
  hipError_t e;
  if (bp.wide) {
    // the tail share evens out the two walks when all their workgroups run
    // side by side; past one round of the CUs it only adds the carry-only
    // chunks (B32 T2048 H16: 742 us with it, 699 us without)
    const bool one_round = 2LL * p.max_items * a.H <= target_workgroups();
    e = launch_bwd_wide(p, a, dec, pair ? 1 : 0, !hp.segmented,
                        one_round ? bwd_tail_q16(a.dk_dim) : 0, s);
  } else {
    e = hp.fast ? launch_bwd_mfma(bp.dvt, p, a, dec, s) : launch_bwd_valu(dt, p, a, dec, s);
  }
  if (e != hipSuccess) return GLA_ERR_HIP;
  return GLA_OK;
}

}  // namespace

extern "C" {

int gla_abi_version(void) { return GLA_ABI_VERSION; }

const char *gla_status_str(gla_status s) {
  switch (s) {
    case GLA_OK: return "ok";
    case GLA_ERR_NULL: return "a required pointer is NULL";
    case GLA_ERR_SHAPE: return "a size is out of range or sizes are inconsistent";
    case GLA_ERR_DTYPE: return "unknown dtype";
    case GLA_ERR_DECAY: return "a decay is not finite or not in (0, 1]";
    case GLA_ERR_ALIAS: return "an output overlaps an input it may not overlap";
    case GLA_ERR_UNSUPPORTED: return "unsupported head count, head size or chunk";
    case GLA_ERR_WORKSPACE: return "workspace missing or too small";
    case GLA_ERR_HIP: return "a HIP kernel launch failed";
    case GLA_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case GLA_ERR_TOO_LARGE:
      return "the call needs more scratch than the allocation-free entry point holds";
    case GLA_STATUS_RANGE_:
    case GLA_STATUS_RANGE_MIN_:
      break;
  }
  return "unknown status";
}

size_t gla_chunk_fwd_workspace_bytes(gla_dtype dt, int B, int T, int H, int dk,
                                     int dv, int chunk) {
  if (check_common(dt, H, dk, dv, chunk) != GLA_OK || B < 1 || T < 0 ||
      (long long)B * T > kMaxTokens)
    return 0;
  return plan_fwd_fixed(dt, B, T, H, dk, dv, chunk).ws_bytes;
}

}  // extern "C"

namespace {

// gla_chunk_fwd, with the output gate when gate != kGateNone (g: o's layout
// and dtype)
gla_status fwd_fixed(int dt, int B, int T, int H, int dk, int dv, int chunk, const void *q,
                     const void *k, const void *v, const void *g, int gate,
                     const float *decay_host, float scale, const float *s0, void *o,
                     float *s_final, void *workspace, size_t workspace_bytes, void *stream) {
  gla_status st = check_common(dt, H, dk, dv, chunk);
  if (st != GLA_OK) return st;
  st = check_gate(gate);
  if (st != GLA_OK) return st;
  if (B < 1 || T < 0 || (long long)B * T > kMaxTokens) return GLA_ERR_SHAPE;
  if (!isfinite(scale)) return GLA_ERR_SHAPE;
  st = check_decay(decay_host, H);
  if (st != GLA_OK) return st;
  const long long tok = (long long)B * T;
  if (tok > 0 && (!q || !k || !v || !o)) return GLA_ERR_NULL;
  if (gate != kGateNone && tok > 0 && !g) return GLA_ERR_NULL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) ||
      misaligned(s0) || misaligned(s_final) || misaligned(g))
    return GLA_ERR_ALIGN;
  const size_t es = elem_size(dt);
  const size_t nqk = (size_t)tok * H * dk * es, nv = (size_t)tok * H * dv * es;
  const size_t ns = (size_t)B * H * dk * dv * sizeof(float);
  const size_t ng = gate != kGateNone ? nv : 0;
  if (overlap(o, nv, q, nqk) || overlap(o, nv, k, nqk) || overlap(o, nv, v, nv) ||
      overlap(o, nv, s0, ns) || overlap(o, nv, g, ng))
    return GLA_ERR_ALIAS;
  if (s_final) {
    if (s_final != s0 && overlap(s_final, ns, s0, ns)) return GLA_ERR_ALIAS;
    if (overlap(s_final, ns, q, nqk) || overlap(s_final, ns, k, nqk) ||
        overlap(s_final, ns, v, nv) || overlap(s_final, ns, o, nv) ||
        overlap(s_final, ns, g, ng))
      return GLA_ERR_ALIAS;
  }
  const HostPlan hp = plan_fwd_fixed(dt, B, T, H, dk, dv, chunk);
  if (hp.ws_bytes > 0) {
    if (!workspace || workspace_bytes < hp.ws_bytes) return GLA_ERR_WORKSPACE;
    if (misaligned(workspace)) return GLA_ERR_ALIGN;
    if (overlap(workspace, hp.ws_bytes, q, nqk) || overlap(workspace, hp.ws_bytes, k, nqk) ||
        overlap(workspace, hp.ws_bytes, v, nv) || overlap(workspace, hp.ws_bytes, o, nv) ||
        overlap(workspace, hp.ws_bytes, s0, ns) || overlap(workspace, hp.ws_bytes, s_final, ns) ||
        overlap(workspace, hp.ws_bytes, g, ng))
      return GLA_ERR_ALIAS;
  }
  hipStream_t s = (hipStream_t)stream;
  if (tok == 0) {
    if (s_final && s_final != s0) {
      (void)hipGetLastError();
      if (launch_state_fill(B, H, dk, dv, s0, s_final, s) != hipSuccess) return GLA_ERR_HIP;
    }
    return GLA_OK;
  }
  FwdArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q; a.k = k; a.v = v; a.o = o; a.s0 = s0; a.s_final = s_final;
  a.scale = scale; a.H = H; a.dk = dk; a.dv = dv;
  a.g = g; a.gate = gate;
  return run_forward(dt, hp, a, make_decay(decay_host, H), workspace, s);
}

}  // namespace

extern "C" {

gla_status gla_chunk_fwd(gla_dtype dt, int B, int T, int H, int dk, int dv,
                         int chunk, const void *q, const void *k,
                         const void *v, const float *decay_host, float scale,
                         const float *s0, void *o, float *s_final,
                         void *workspace, size_t workspace_bytes,
                         void *stream) {
  return fwd_fixed(dt, B, T, H, dk, dv, chunk, q, k, v, nullptr, kGateNone, decay_host,
                   scale, s0, o, s_final, workspace, workspace_bytes, stream);
}

gla_status gla_chunk_fwd_gated(gla_dtype dt, int B, int T, int H, int dk, int dv,
                               int chunk, const void *q, const void *k, const void *v,
                               const void *g, gla_gate gate, const float *decay_host,
                               float scale, const float *s0, void *o, float *s_final,
                               void *workspace, size_t workspace_bytes, void *stream) {
  return fwd_fixed(dt, B, T, H, dk, dv, chunk, q, k, v, g, gate_code(gate), decay_host,
                   scale, s0, o, s_final, workspace, workspace_bytes, stream);
}


size_t gla_linear_attn_fwd_workspace_bytes(gla_dtype dt, int B, int T, int H,
                                           int dk, int dv, int chunk) {
  if (check_common(dt, H, dk, dv, chunk) != GLA_OK || B < 1 || T < 0 ||
      (long long)B * T > kMaxTokens)
    return 0;
  return plan_linear_attn(dt, B, T, H, dk, dv, chunk).ws_bytes;
}

gla_status gla_linear_attn_fwd(gla_dtype dt, int B, int T, int H, int dk, int dv,
                               int chunk, const void *q, const void *k, const void *v,
                               const float *s0, const float *z0, void *o,
                               float *s_final, float *z_final, void *workspace,
                               size_t workspace_bytes, void *stream) {
  gla_status st = check_common(dt, H, dk, dv, chunk);
  if (st != GLA_OK) return st;
  if (B < 1 || T < 0 || (long long)B * T > kMaxTokens) return GLA_ERR_SHAPE;
  const long long tok = (long long)B * T;
  if (tok > 0 && (!q || !k || !v || !o)) return GLA_ERR_NULL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) ||
      misaligned(s0) || misaligned(s_final) || misaligned(z0) || misaligned(z_final))
    return GLA_ERR_ALIGN;
  const size_t es = elem_size(dt);
  const size_t nqk = (size_t)tok * H * dk * es, nv = (size_t)tok * H * dv * es;
  const size_t ns = (size_t)B * H * dk * dv * sizeof(float);
  const size_t nz = (size_t)B * H * dk * sizeof(float);
  // every output range (o, s_final, z_final) must be disjoint from every
  // other range, inputs included (no in-place final state here)
  const void *rp[7] = {q, k, v, s0, z0, o, s_final};
  const size_t rn[7] = {nqk, nqk, nv, ns, nz, nv, ns};
  for (int i = 0; i < 7; ++i) {
    if (i != 5 && overlap(o, nv, rp[i], rn[i])) return GLA_ERR_ALIAS;
    if (s_final && i != 6 && overlap(s_final, ns, rp[i], rn[i])) return GLA_ERR_ALIAS;
    if (z_final && overlap(z_final, nz, rp[i], rn[i])) return GLA_ERR_ALIAS;
  }
  const HostPlan hp = plan_linear_attn(dt, B, T, H, dk, dv, chunk);
  if (hp.ws_bytes > 0) {
    if (!workspace || workspace_bytes < hp.ws_bytes) return GLA_ERR_WORKSPACE;
    if (misaligned(workspace)) return GLA_ERR_ALIGN;
    for (int i = 0; i < 7; ++i)
      if (overlap(workspace, hp.ws_bytes, rp[i], rn[i])) return GLA_ERR_ALIAS;
    if (overlap(workspace, hp.ws_bytes, z_final, nz)) return GLA_ERR_ALIAS;
  }
  hipStream_t s = (hipStream_t)stream;
  if (tok == 0) {
    if (s_final || z_final) (void)hipGetLastError();
    if (s_final && launch_state_fill(B, H, dk, dv, s0, s_final, s) != hipSuccess)
      return GLA_ERR_HIP;
    if (z_final && launch_state_fill(B, H, dk, 1, z0, z_final, s) != hipSuccess)
      return GLA_ERR_HIP;
    return GLA_OK;
  }
  FwdArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q; a.k = k; a.v = v; a.o = o; a.s0 = s0; a.s_final = s_final;
  a.scale = 1.0f; a.H = H; a.dk = dk; a.dv = dv;
  a.norm = 1; a.z0 = z0; a.z_final = z_final;
  return run_forward(dt, hp, a, unit_decay(), workspace, s);
}

size_t gla_linear_attn_fwd_varlen_workspace_bytes(gla_dtype dt, int N, int total_T,
                                                  int H, int dk, int dv, int chunk) {
  if (check_common(dt, H, dk, dv, chunk) != GLA_OK || N < 1 || total_T < 0) return 0;
  return plan_linear_attn_varlen(dt, N, total_T, H, dk, dv, chunk).ws_bytes;
}

gla_status gla_linear_attn_fwd_varlen(gla_dtype dt, int N, int total_T, int H, int dk,
                                      int dv, int chunk, const int32_t *cu_seqlens,
                                      const void *q, const void *k, const void *v,
                                      const float *s0, const float *z0, void *o,
                                      float *s_final, float *z_final, void *workspace,
                                      size_t workspace_bytes, void *stream) {
  gla_status st = check_common(dt, H, dk, dv, chunk);
  if (st != GLA_OK) return st;
  if (N < 1 || total_T < 0 || N > (1 << 28)) return GLA_ERR_SHAPE;
  if (!cu_seqlens) return GLA_ERR_NULL;
  if (total_T > 0 && (!q || !k || !v || !o)) return GLA_ERR_NULL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) ||
      misaligned(s0) || misaligned(s_final) || misaligned(z0) || misaligned(z_final) ||
      ((uintptr_t)cu_seqlens & 3u))
    return GLA_ERR_ALIGN;
  const size_t es = elem_size(dt);
  const size_t nqk = (size_t)total_T * H * dk * es, nv = (size_t)total_T * H * dv * es;
  const size_t ns = (size_t)N * H * dk * dv * sizeof(float);
  const size_t nz = (size_t)N * H * dk * sizeof(float);
  const size_t ncu = sizeof(int32_t) * ((size_t)N + 1);
  const void *rp[8] = {q, k, v, s0, z0, cu_seqlens, o, s_final};
  const size_t rn[8] = {nqk, nqk, nv, ns, nz, ncu, nv, ns};
  for (int i = 0; i < 8; ++i) {
    if (i != 6 && overlap(o, nv, rp[i], rn[i])) return GLA_ERR_ALIAS;
    if (s_final && i != 7 && overlap(s_final, ns, rp[i], rn[i])) return GLA_ERR_ALIAS;
    if (z_final && overlap(z_final, nz, rp[i], rn[i])) return GLA_ERR_ALIAS;
  }
  HostPlan hp = plan_linear_attn_varlen(dt, N, total_T, H, dk, dv, chunk);
  if (hp.ws_bytes > 0) {
    if (!workspace || workspace_bytes < hp.ws_bytes) return GLA_ERR_WORKSPACE;
    if (misaligned(workspace)) return GLA_ERR_ALIGN;
    for (int i = 0; i < 8; ++i)
      if (overlap(workspace, hp.ws_bytes, rp[i], rn[i])) return GLA_ERR_ALIAS;
    if (overlap(workspace, hp.ws_bytes, z_final, nz)) return GLA_ERR_ALIAS;
  }
  hipStream_t s = (hipStream_t)stream;
  if (total_T == 0) {
    if (s_final || z_final) (void)hipGetLastError();
    if (s_final && launch_state_fill(N, H, dk, dv, s0, s_final, s) != hipSuccess)
      return GLA_ERR_HIP;
    if (z_final && launch_state_fill(N, H, dk, 1, z0, z_final, s) != hipSuccess)
      return GLA_ERR_HIP;
    return GLA_OK;
  }
  hp.p.cu = cu_seqlens;
  FwdArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q; a.k = k; a.v = v; a.o = o; a.s0 = s0; a.s_final = s_final;
  a.scale = 1.0f; a.H = H; a.dk = dk; a.dv = dv;
  a.norm = 1; a.z0 = z0; a.z_final = z_final;
  return run_forward(dt, hp, a, unit_decay(), workspace, s);
}

size_t gla_chunk_fwd_varlen_workspace_bytes(gla_dtype dt, int N, int total_T,
                                            int H, int dk, int dv, int chunk) {
  if (check_common(dt, H, dk, dv, chunk) != GLA_OK || N < 1 || total_T < 0)
    return 0;
  return plan_varlen(dt, N, total_T, H, dk, dv, chunk).ws_bytes;
}

}  // extern "C"

namespace {

// ---------------------------------------------------------------------------
// Fixed scratch of the allocation-free entry point: one array per GPU, for
// the life of the process, so that a call needs no hipMalloc. The name
// `scratch` is a host-side stand-in in host code; the device address of each
// GPU's copy comes from hipGetSymbolAddress with that GPU current, once per
// device, and only that address is ever handed to kernels.
// ---------------------------------------------------------------------------
constexpr size_t kNoAllocScratchBytes = GLA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void *scratch_dev[kMaxDevices];  // device address of `scratch` per device, or null

// The scratch of the device that stream `s` belongs to (the current device
// for the null stream). The first call on a device looks the array's
// address up with that device current, switching to it for the lookup if
// the caller's current device is another one.
hipError_t noalloc_scratch(hipStream_t s, void **ptr) {
  int dev = 0;
  hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_dev[dev]) {
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t back = hipSetDevice(cur);
      if (e == hipSuccess) e = back;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    scratch_dev[dev] = p;
  }
  *ptr = scratch_dev[dev];
  return hipSuccess;
}

// gla_chunk_fwd_varlen with the workspace given (noalloc false), or taken
// from this device's fixed scratch array (noalloc true: workspace and
// workspace_bytes are ignored).
gla_status fwd_varlen(int dt, int N, int total_T, int H, int dk, int dv, int chunk,
                      const int32_t *cu_seqlens, const void *q, const void *k,
                      const void *v, const void *g, int gate, const float *decay_host,
                      float scale, const float *s0, void *o, float *s_final, void *workspace,
                      size_t workspace_bytes, void *stream, bool noalloc) {
  gla_status st = check_common(dt, H, dk, dv, chunk);
  if (st != GLA_OK) return st;
  st = check_gate(gate);
  if (st != GLA_OK) return st;
  if (N < 1 || total_T < 0 || N > (1 << 28)) return GLA_ERR_SHAPE;
  if (!isfinite(scale)) return GLA_ERR_SHAPE;
  st = check_decay(decay_host, H);
  if (st != GLA_OK) return st;
  if (!cu_seqlens) return GLA_ERR_NULL;
  if (total_T > 0 && (!q || !k || !v || !o)) return GLA_ERR_NULL;
  if (gate != kGateNone && total_T > 0 && !g) return GLA_ERR_NULL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) ||
      misaligned(s0) || misaligned(s_final) || misaligned(g) || ((uintptr_t)cu_seqlens & 3u))
    return GLA_ERR_ALIGN;
  const size_t es = elem_size(dt);
  const size_t nqk = (size_t)total_T * H * dk * es, nv = (size_t)total_T * H * dv * es;
  const size_t ns = (size_t)N * H * dk * dv * sizeof(float);
  const size_t ncu = sizeof(int32_t) * ((size_t)N + 1);
  const size_t ng = gate != kGateNone ? nv : 0;
  if (overlap(o, nv, q, nqk) || overlap(o, nv, k, nqk) || overlap(o, nv, v, nv) ||
      overlap(o, nv, s0, ns) || overlap(o, nv, cu_seqlens, ncu) || overlap(o, nv, g, ng))
    return GLA_ERR_ALIAS;
  if (s_final) {
    if (s_final != s0 && overlap(s_final, ns, s0, ns)) return GLA_ERR_ALIAS;
    if (overlap(s_final, ns, q, nqk) || overlap(s_final, ns, k, nqk) ||
        overlap(s_final, ns, v, nv) || overlap(s_final, ns, o, nv) ||
        overlap(s_final, ns, cu_seqlens, ncu) || overlap(s_final, ns, g, ng))
      return GLA_ERR_ALIAS;
  }
  const HostPlan hp = plan_varlen(dt, N, total_T, H, dk, dv, chunk);
  if (noalloc) {
    // every check above is done; the scratch lookup is the first HIP call
    if (hp.ws_bytes > kNoAllocScratchBytes) return GLA_ERR_TOO_LARGE;
    workspace = nullptr;
    workspace_bytes = 0;
    if (hp.ws_bytes > 0) {
      if (noalloc_scratch((hipStream_t)stream, &workspace) != hipSuccess) return GLA_ERR_HIP;
      workspace_bytes = kNoAllocScratchBytes;
    }
  }
  if (hp.ws_bytes > 0) {
    if (!workspace || workspace_bytes < hp.ws_bytes) return GLA_ERR_WORKSPACE;
    if (misaligned(workspace)) return GLA_ERR_ALIGN;
    if (overlap(workspace, hp.ws_bytes, q, nqk) || overlap(workspace, hp.ws_bytes, k, nqk) ||
        overlap(workspace, hp.ws_bytes, v, nv) || overlap(workspace, hp.ws_bytes, o, nv) ||
        overlap(workspace, hp.ws_bytes, s0, ns) || overlap(workspace, hp.ws_bytes, s_final, ns) ||
        overlap(workspace, hp.ws_bytes, cu_seqlens, ncu) || overlap(workspace, hp.ws_bytes, g, ng))
      return GLA_ERR_ALIAS;
  }
  hipStream_t s = (hipStream_t)stream;
  if (total_T == 0) {
    if (s_final && s_final != s0) {
      (void)hipGetLastError();
      if (launch_state_fill(N, H, dk, dv, s0, s_final, s) != hipSuccess) return GLA_ERR_HIP;
    }
    return GLA_OK;
  }
  Plan p = hp.p;
  p.cu = cu_seqlens;
  HostPlan hq = hp;
  hq.p = p;
  FwdArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q; a.k = k; a.v = v; a.o = o; a.s0 = s0; a.s_final = s_final;
  a.scale = scale; a.H = H; a.dk = dk; a.dv = dv;
  a.g = g; a.gate = gate;
  return run_forward(dt, hq, a, make_decay(decay_host, H), workspace, s);
}

}  // namespace

extern "C" {

gla_status gla_chunk_fwd_varlen(gla_dtype dt, int N, int total_T, int H,
                                int dk, int dv, int chunk,
                                const int32_t *cu_seqlens, const void *q,
                                const void *k, const void *v,
                                const float *decay_host, float scale,
                                const float *s0, void *o, float *s_final,
                                void *workspace, size_t workspace_bytes,
                                void *stream) {
  return fwd_varlen(dt, N, total_T, H, dk, dv, chunk, cu_seqlens, q, k, v, nullptr, kGateNone,
                    decay_host, scale, s0, o, s_final, workspace, workspace_bytes, stream, false);
}

gla_status gla_chunk_fwd_varlen_gated(gla_dtype dt, int N, int total_T, int H, int dk, int dv,
                                      int chunk, const int32_t *cu_seqlens, const void *q,
                                      const void *k, const void *v, const void *g,
                                      gla_gate gate, const float *decay_host, float scale,
                                      const float *s0, void *o, float *s_final,
                                      void *workspace, size_t workspace_bytes, void *stream) {
  return fwd_varlen(dt, N, total_T, H, dk, dv, chunk, cu_seqlens, q, k, v, g, gate_code(gate),
                    decay_host, scale, s0, o, s_final, workspace, workspace_bytes, stream, false);
}

gla_status gla_chunk_fwd_varlen_noalloc(gla_dtype dt, int N, int total_T, int H,
                                        int dk, int dv, int chunk,
                                        const int32_t *cu_seqlens, const void *q,
                                        const void *k, const void *v,
                                        const float *decay_host, float scale,
                                        const float *s0, void *o, float *s_final,
                                        void *stream) {
  return fwd_varlen(dt, N, total_T, H, dk, dv, chunk, cu_seqlens, q, k, v, nullptr, kGateNone,
                    decay_host, scale, s0, o, s_final, nullptr, 0, stream, true);
}

size_t gla_chunk_bwd_workspace_bytes(gla_dtype dt, int B, int T, int H, int dk,
                                     int dv, int chunk) {
  if (check_common(dt, H, dk, dv, chunk) != GLA_OK ||
      B < 1 || T < 0 || (long long)B * T > kMaxTokens)
    return 0;
  const HostPlan hp =
      bwd_plan_fixed(dt, B, T, H, dk, dv, chunk);
  return bwd_layout(hp, (long long)B * T, H, dk, dv).ws_bytes;
}

gla_status gla_chunk_bwd(gla_dtype dt, int B, int T, int H, int dk, int dv,
                         int chunk, const void *q, const void *k, const void *v,
                         const float *decay_host, float scale, const float *s0,
                         const void *dout, const float *ds_final, void *dq,
                         void *dk_out, void *dv_out, float *ds0, void *workspace,
                         size_t workspace_bytes, void *stream) {
  gla_status st = check_common(dt, H, dk, dv, chunk);
  if (st != GLA_OK) return st;
  if (B < 1 || T < 0 || (long long)B * T > kMaxTokens) return GLA_ERR_SHAPE;
  if (!isfinite(scale)) return GLA_ERR_SHAPE;
  st = check_decay(decay_host, H);
  if (st != GLA_OK) return st;
  const long long tok = (long long)B * T;
  if (tok > 0 && (!q || !k || !v || !dout || !dq || !dk_out || !dv_out)) return GLA_ERR_NULL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(dout) ||
      misaligned(dq) || misaligned(dk_out) || misaligned(dv_out) || misaligned(s0) ||
      misaligned(ds_final) || misaligned(ds0))
    return GLA_ERR_ALIGN;
  const size_t es = elem_size(dt);
  const size_t nqk = (size_t)tok * H * dk * es, nv = (size_t)tok * H * dv * es;
  const size_t ns = (size_t)B * H * dk * dv * sizeof(float);
  // outputs overlap no input and no other output
  const void *in[6] = {q, k, v, dout, s0, ds_final};
  const size_t in_n[6] = {nqk, nqk, nv, nv, ns, ns};
  const void *out[4] = {dq, dk_out, dv_out, ds0};
  const size_t out_n[4] = {nqk, nqk, nv, ns};
  for (int a = 0; a < 4; ++a) {
    for (int b = 0; b < 6; ++b)
      if (overlap(out[a], out_n[a], in[b], in_n[b])) return GLA_ERR_ALIAS;
    for (int b = a + 1; b < 4; ++b)
      if (overlap(out[a], out_n[a], out[b], out_n[b])) return GLA_ERR_ALIAS;
  }
  const BwdPlan bp = bwd_layout(
      bwd_plan_fixed(dt, B, T, H, dk, dv, chunk), tok, H,
      dk, dv);
  if (bp.ws_bytes > 0) {
    if (!workspace || workspace_bytes < bp.ws_bytes) return GLA_ERR_WORKSPACE;
    if (misaligned(workspace)) return GLA_ERR_ALIGN;
    for (int b = 0; b < 6; ++b)
      if (overlap(workspace, bp.ws_bytes, in[b], in_n[b])) return GLA_ERR_ALIAS;
    for (int a = 0; a < 4; ++a)
      if (overlap(workspace, bp.ws_bytes, out[a], out_n[a])) return GLA_ERR_ALIAS;
  }
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  if (tok == 0) {  // no tokens: the gradient passes straight through
    if (ds0 && launch_state_fill(B, H, dk, dv, ds_final, ds0, s) != hipSuccess)
      return GLA_ERR_HIP;
    return GLA_OK;
  }
  BwdArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q; a.k = k; a.v = v; a.dout = dout; a.s0 = s0; a.ds_final = ds_final;
  a.dq = dq; a.dk = dk_out; a.dv_out = dv_out; a.ds0 = ds0;
  a.scale = scale; a.H = H; a.dv = dv; a.dk_dim = dk;
  return run_backward(dt, bp, a, make_decay(decay_host, H), workspace, s);
}

size_t gla_chunk_bwd_varlen_workspace_bytes(gla_dtype dt, int N, int total_T, int H,
                                            int dk, int dv, int chunk) {
  if (check_common(dt, H, dk, dv, chunk) != GLA_OK ||
      N < 1 || N > (1 << 28) || total_T < 0)
    return 0;
  const HostPlan hp =
      bwd_plan_varlen(dt, N, total_T, H, dk, dv, chunk);
  return bwd_layout(hp, total_T, H, dk, dv).ws_bytes;
}

gla_status gla_chunk_bwd_varlen(gla_dtype dt, int N, int total_T, int H, int dk,
                                int dv, int chunk, const int32_t *cu_seqlens,
                                const void *q, const void *k, const void *v,
                                const float *decay_host, float scale, const float *s0,
                                const void *dout, const float *ds_final, void *dq,
                                void *dk_out, void *dv_out, float *ds0, void *workspace,
                                size_t workspace_bytes, void *stream) {
  gla_status st = check_common(dt, H, dk, dv, chunk);
  if (st != GLA_OK) return st;
  if (N < 1 || N > (1 << 28) || total_T < 0) return GLA_ERR_SHAPE;
  if (!isfinite(scale)) return GLA_ERR_SHAPE;
  st = check_decay(decay_host, H);
  if (st != GLA_OK) return st;
  if (!cu_seqlens) return GLA_ERR_NULL;
  if (total_T > 0 && (!q || !k || !v || !dout || !dq || !dk_out || !dv_out)) return GLA_ERR_NULL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(dout) ||
      misaligned(dq) || misaligned(dk_out) || misaligned(dv_out) || misaligned(s0) ||
      misaligned(ds_final) || misaligned(ds0) || ((uintptr_t)cu_seqlens & 3u))
    return GLA_ERR_ALIGN;
  const size_t es = elem_size(dt);
  const size_t nqk = (size_t)total_T * H * dk * es, nv = (size_t)total_T * H * dv * es;
  const size_t ns = (size_t)N * H * dk * dv * sizeof(float);
  const size_t ncu = sizeof(int32_t) * ((size_t)N + 1);
  const void *in[7] = {q, k, v, dout, s0, ds_final, cu_seqlens};
  const size_t in_n[7] = {nqk, nqk, nv, nv, ns, ns, ncu};
  const void *out[4] = {dq, dk_out, dv_out, ds0};
  const size_t out_n[4] = {nqk, nqk, nv, ns};
  for (int a = 0; a < 4; ++a) {
    for (int b = 0; b < 7; ++b)
      if (overlap(out[a], out_n[a], in[b], in_n[b])) return GLA_ERR_ALIAS;
    for (int b = a + 1; b < 4; ++b)
      if (overlap(out[a], out_n[a], out[b], out_n[b])) return GLA_ERR_ALIAS;
  }
  HostPlan hp =
      bwd_plan_varlen(dt, N, total_T, H, dk, dv, chunk);
  hp.p.cu = cu_seqlens;
  const BwdPlan bp = bwd_layout(hp, total_T, H, dk, dv);
  if (bp.ws_bytes > 0) {
    if (!workspace || workspace_bytes < bp.ws_bytes) return GLA_ERR_WORKSPACE;
    if (misaligned(workspace)) return GLA_ERR_ALIGN;
    for (int b = 0; b < 7; ++b)
      if (overlap(workspace, bp.ws_bytes, in[b], in_n[b])) return GLA_ERR_ALIAS;
    for (int a = 0; a < 4; ++a)
      if (overlap(workspace, bp.ws_bytes, out[a], out_n[a])) return GLA_ERR_ALIAS;
  }
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  if (total_T == 0) {  // no tokens: the gradient passes straight through
    if (ds0 && launch_state_fill(N, H, dk, dv, ds_final, ds0, s) != hipSuccess)
      return GLA_ERR_HIP;
    return GLA_OK;
  }
  BwdArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q; a.k = k; a.v = v; a.dout = dout; a.s0 = s0; a.ds_final = ds_final;
  a.dq = dq; a.dk = dk_out; a.dv_out = dv_out; a.ds0 = ds0;
  a.scale = scale; a.H = H; a.dv = dv; a.dk_dim = dk;
  return run_backward(dt, bp, a, make_decay(decay_host, H), workspace, s);
}

gla_status gla_short_conv_fwd(gla_dtype dt, int B, int T, int D, const void *x,
                              const float *w, const float *bias, const float *window_in,
                              void *y, float *window_out, void *stream) {
  if (dt != GLA_F32 && dt != GLA_BF16) return GLA_ERR_DTYPE;
  if (B < 1 || T < 0 || D < 1 || (long long)B * T > kMaxTokens) return GLA_ERR_SHAPE;
  if (D % 8 != 0 || D > (1 << 20)) return GLA_ERR_UNSUPPORTED;
  if (!w || (T > 0 && (!x || !y))) return GLA_ERR_NULL;
  if (misaligned(x) || misaligned(y) || misaligned(window_in) || misaligned(window_out) ||
      misaligned(w) || ((uintptr_t)bias & 3u))
    return GLA_ERR_ALIGN;
  const size_t es = elem_size(dt);
  const size_t nx = (size_t)B * T * D * es, nwin = (size_t)B * 4 * D * sizeof(float);
  const size_t nw = (size_t)D * 4 * sizeof(float), nb = (size_t)D * sizeof(float);
  const void *in[5] = {x, w, bias, window_in, nullptr};
  const size_t in_n[5] = {nx, nw, nb, nwin, 0};
  for (int i = 0; i < 4; ++i)
    if (overlap(y, nx, in[i], in_n[i]) || overlap(window_out, nwin, in[i], in_n[i]))
      return GLA_ERR_ALIAS;
  if (overlap(y, nx, window_out, nwin)) return GLA_ERR_ALIAS;
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  if (T == 0) {  // no tokens: the window passes through
    if (window_out && launch_state_fill(B, 1, 4, D, window_in, window_out, s) != hipSuccess)
      return GLA_ERR_HIP;
    return GLA_OK;
  }
  if (launch_short_conv_fwd(dt, B, T, D, x, w, bias, window_in, y, window_out, s) != hipSuccess)
    return GLA_ERR_HIP;
  return GLA_OK;
}

gla_status gla_short_conv_decode_step(gla_dtype dt, int N, int D, const void *x,
                                      const float *w, const float *bias, float *window,
                                      void *y, void *stream) {
  if (dt != GLA_F32 && dt != GLA_BF16) return GLA_ERR_DTYPE;
  if (N < 0 || D < 1) return GLA_ERR_SHAPE;
  if (D % 8 != 0 || D > (1 << 20)) return GLA_ERR_UNSUPPORTED;
  if (N == 0) return GLA_OK;
  if (!x || !w || !window || !y) return GLA_ERR_NULL;
  if (misaligned(x) || misaligned(y) || misaligned(window) || misaligned(w) ||
      ((uintptr_t)bias & 3u))
    return GLA_ERR_ALIGN;
  const size_t es = elem_size(dt);
  const size_t nx = (size_t)N * D * es, nwin = (size_t)N * 4 * D * sizeof(float);
  const size_t nw = (size_t)D * 4 * sizeof(float), nb = (size_t)D * sizeof(float);
  if (overlap(window, nwin, x, nx) || overlap(window, nwin, w, nw) ||
      overlap(window, nwin, bias, nb) || overlap(window, nwin, y, nx) ||
      overlap(y, nx, x, nx) || overlap(y, nx, w, nw) || overlap(y, nx, bias, nb))
    return GLA_ERR_ALIAS;
  (void)hipGetLastError();
  if (launch_short_conv_decode(dt, N, D, x, w, bias, window, y, (hipStream_t)stream) != hipSuccess)
    return GLA_ERR_HIP;
  return GLA_OK;
}

}  // extern "C"

namespace {

// gla_decode_step, with the output gate when gate != kGateNone (g [N, H, dv]
// in o's dtype)
gla_status decode_step(int dt, int N, int H, int dk, int dv, const void *q, const void *k,
                       const void *v, const void *g, int gate, const float *decay_host,
                       float scale, float *state, void *o, void *stream) {
  gla_status st = check_common(dt, H, dk, dv, 0);
  if (st != GLA_OK) return st;
  st = check_gate(gate);
  if (st != GLA_OK) return st;
  if (N < 0 || (long long)N * H > kMaxTokens) return GLA_ERR_SHAPE;
  if (!isfinite(scale)) return GLA_ERR_SHAPE;
  st = check_decay(decay_host, H);
  if (st != GLA_OK) return st;
  if (N == 0) return GLA_OK;
  if (!q || !k || !v || !o || !state) return GLA_ERR_NULL;
  if (gate != kGateNone && !g) return GLA_ERR_NULL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) || misaligned(state) ||
      misaligned(g))
    return GLA_ERR_ALIGN;
  const size_t es = elem_size(dt);
  const size_t nqk = (size_t)N * H * dk * es, nv = (size_t)N * H * dv * es;
  const size_t ns = (size_t)N * H * dk * dv * sizeof(float);
  const size_t ng = gate != kGateNone ? nv : 0;
  if (overlap(state, ns, q, nqk) || overlap(state, ns, k, nqk) ||
      overlap(state, ns, v, nv) || overlap(state, ns, o, nv) || overlap(state, ns, g, ng) ||
      overlap(o, nv, q, nqk) || overlap(o, nv, k, nqk) || overlap(o, nv, v, nv) ||
      overlap(o, nv, g, ng))
    return GLA_ERR_ALIAS;
  (void)hipGetLastError();
  if (launch_decode(dt, N, H, dk, dv, q, k, v, make_decay(decay_host, H), scale,
                    state, o, (hipStream_t)stream, nullptr, 0, nullptr, g, gate) != hipSuccess)
    return GLA_ERR_HIP;
  return GLA_OK;
}

}  // namespace

extern "C" {

gla_status gla_decode_step(gla_dtype dt, int N, int H, int dk, int dv,
                           const void *q, const void *k, const void *v,
                           const float *decay_host, float scale, float *state,
                           void *o, void *stream) {
  return decode_step(dt, N, H, dk, dv, q, k, v, nullptr, kGateNone, decay_host, scale, state,
                     o, stream);
}

gla_status gla_decode_step_gated(gla_dtype dt, int N, int H, int dk, int dv, const void *q,
                                 const void *k, const void *v, const void *g, gla_gate gate,
                                 const float *decay_host, float scale, float *state, void *o,
                                 void *stream) {
  return decode_step(dt, N, H, dk, dv, q, k, v, g, gate_code(gate), decay_host, scale, state,
                     o, stream);
}

gla_status gla_linear_attn_decode_step(gla_dtype dt, int N, int H, int dk, int dv,
                                       const void *q, const void *k, const void *v,
                                       float *state, float *z, void *o, void *stream) {
  gla_status st = check_common(dt, H, dk, dv, 0);
  if (st != GLA_OK) return st;
  if (N < 0 || (long long)N * H > kMaxTokens) return GLA_ERR_SHAPE;
  if (N == 0) return GLA_OK;
  if (!q || !k || !v || !o || !state || !z) return GLA_ERR_NULL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) || misaligned(state) ||
      misaligned(z))
    return GLA_ERR_ALIGN;
  const size_t es = elem_size(dt);
  const size_t nqk = (size_t)N * H * dk * es, nv = (size_t)N * H * dv * es;
  const size_t ns = (size_t)N * H * dk * dv * sizeof(float), nz = (size_t)N * H * dk * 4;
  const void *rp[6] = {q, k, v, o, state, z};
  const size_t rn[6] = {nqk, nqk, nv, nv, ns, nz};
  for (int a = 3; a < 6; ++a)  // o, state, z: disjoint from everything else
    for (int b = 0; b < 6; ++b)
      if (a != b && overlap(rp[a], rn[a], rp[b], rn[b])) return GLA_ERR_ALIAS;
  (void)hipGetLastError();
  if (launch_decode(dt, N, H, dk, dv, q, k, v, unit_decay(), 1.0f, state, o, (hipStream_t)stream,
                    nullptr, 0, z) != hipSuccess)
    return GLA_ERR_HIP;
  return GLA_OK;
}

gla_status gla_decode_step_pool(gla_dtype dt, int N, int H, int dk, int dv,
                                const void *q, const void *k, const void *v,
                                const float *decay_host, float scale,
                                const int32_t *slots, int pool_size,
                                float *state_pool, void *o, void *stream) {
  gla_status st = check_common(dt, H, dk, dv, 0);
  if (st != GLA_OK) return st;
  if (N < 0 || (long long)N * H > kMaxTokens) return GLA_ERR_SHAPE;
  if (pool_size < 1 || (long long)pool_size * H > kMaxTokens) return GLA_ERR_SHAPE;
  if (!isfinite(scale)) return GLA_ERR_SHAPE;
  st = check_decay(decay_host, H);
  if (st != GLA_OK) return st;
  if (N == 0) return GLA_OK;
  if (!q || !k || !v || !o || !state_pool || !slots) return GLA_ERR_NULL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) ||
      misaligned(state_pool) || ((uintptr_t)slots & 3u))
    return GLA_ERR_ALIGN;
  const size_t es = elem_size(dt);
  const size_t nqk = (size_t)N * H * dk * es, nv = (size_t)N * H * dv * es;
  const size_t ns = (size_t)pool_size * H * dk * dv * sizeof(float);
  const size_t nsl = sizeof(int32_t) * (size_t)N;
  if (overlap(state_pool, ns, q, nqk) || overlap(state_pool, ns, k, nqk) ||
      overlap(state_pool, ns, v, nv) || overlap(state_pool, ns, o, nv) ||
      overlap(state_pool, ns, slots, nsl) || overlap(o, nv, q, nqk) ||
      overlap(o, nv, k, nqk) || overlap(o, nv, v, nv) || overlap(o, nv, slots, nsl))
    return GLA_ERR_ALIAS;
  (void)hipGetLastError();
  if (launch_decode(dt, N, H, dk, dv, q, k, v, make_decay(decay_host, H), scale,
                    state_pool, o, (hipStream_t)stream, slots, pool_size) != hipSuccess)
    return GLA_ERR_HIP;
  return GLA_OK;
}

}  // extern "C"
