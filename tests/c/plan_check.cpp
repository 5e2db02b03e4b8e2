// plan_check.cpp -- host-side checks of the library's work planning: time
// segments, packed-sequence items (the device planner replayed on the host),
// the dispatch order's bounds, the workspace layouts and the workgroup ->
// (unit, d_v tile) mapping, for the long-context, packed and ragged plans and
// the head shapes around them.
//
// Built by tests/test_host_sanitizers.py with AddressSanitizer, UBSan and the
// library's debug plan checks (GLA_DEBUG). It makes no HIP call: the
// planners, item decoding and workgroup mapping it exercises are the
// library's own code (gla_api.cpp is compiled into this file; the decoding
// and mapping helpers in gla_device.h are host and device functions).
//
// Usage: plan_check [comma-separated packed lengths ...]   (extra packed
// batches to check besides the built-in ones; exit status 0 when all hold)
#include "gla_api.cpp"
#include "gla_device.h"

#include <stdio.h>
#include <stdlib.h>

#include <array>
#include <string>
#include <vector>

namespace {

int failures = 0;
long long checks = 0;
std::string where;

#define EXPECT(c)                                                                  \
  do {                                                                             \
    ++checks;                                                                      \
    if (!(c)) {                                                                    \
      if (failures < 50)                                                           \
        fprintf(stderr, "plan_check.cpp:%d: %s failed [%s]\n", __LINE__, #c, where.c_str()); \
      ++failures;                                                                  \
    }                                                                              \
  } while (0)

void set_target(long long wgs) {
  if (wgs > 0) {
    char b[32];
    snprintf(b, sizeof b, "%lld", wgs);
    setenv("GLA_TARGET_WGS", b, 1);
  } else {
    unsetenv("GLA_TARGET_WGS");
  }
}

std::vector<int32_t> cu_of(const std::vector<int> &lens) {
  std::vector<int32_t> cu(lens.size() + 1, 0);
  for (size_t n = 0; n < lens.size(); ++n) cu[n + 1] = cu[n] + lens[n];
  return cu;
}

// The device planner (planner_kernel) replayed on the host: sequence n
// becomes ceil(L_n / seg) items of seg tokens (the last one shorter), one
// empty item when L_n = 0; index[0] = item count, index[1 + n] = first item
// of sequence n, index[1 + N] = count.
void host_planner(const Plan &p, const std::vector<int32_t> &cu, std::vector<int32_t> &index,
                  std::vector<int4> &items) {
  const int N = p.n_seq;
  index.assign((size_t)N + 2, 0);
  items.assign((size_t)p.max_items, make_int4(-1, -1, -1, -1));
  int pos = 0;
  for (int n = 0; n < N; ++n) {
    const int a = clampi(cu[n], 0, p.total_T), b = clampi(cu[n + 1], a, p.total_T);
    const int L = b - a;
    const int ns = L > 0 ? (L + p.seg_len - 1) / p.seg_len : 1;
    index[1 + n] = pos < p.max_items ? pos : p.max_items;
    for (int g = 0; g < ns; ++g, ++pos) {
      EXPECT(pos < p.max_items);  // the host bound on items always holds
      if (pos >= p.max_items) continue;
      const int t0 = a + g * p.seg_len, t1 = t0 + p.seg_len < b ? t0 + p.seg_len : b;
      items[pos] = make_int4(n, t0, t1, (g == 0 ? kFirstSeg : 0) | (g == ns - 1 ? kLastSeg : 0));
    }
  }
  index[0] = pos < p.max_items ? pos : p.max_items;
  index[1 + N] = index[0];
}

// Every (unit, d_v tile) with unit < units is produced by exactly one
// workgroup id below the launch's grid; the others fall past the units.
void check_mapping(int deal, long long units, int ndt) {
  Plan p;
  memset(&p, 0, sizeof p);
  p.deal = deal;
  const unsigned grid = xcd_grid(deal, units, ndt);
  EXPECT(grid > 0 && grid < (1u << 31));
  std::vector<unsigned char> seen((size_t)units * ndt, 0);
  for (unsigned P = 0; P < grid; ++P) {
    int unit = -1, dtile = -1;
    xcd_unit_at(p, (int)P, ndt, (int)units, unit, dtile);
    EXPECT(unit >= 0 && dtile >= 0 && dtile < ndt);
    if (unit >= 0 && unit < units && dtile >= 0 && dtile < ndt) {
      EXPECT(seen[(size_t)unit * ndt + dtile] == 0);
      seen[(size_t)unit * ndt + dtile] = 1;
    }
  }
  for (size_t i = 0; i < seen.size(); ++i) EXPECT(seen[i] == 1);
}

// The plan's items tile every sequence exactly and in order, in whole
// chunks from the sequence start, with the right first/last flags; every
// state slot a kernel touches (idx - 1 read by a later segment, idx written
// by the state pass, idx + 1 read by the reverse walk) is inside the slots.
void check_items(Plan p, const std::vector<int32_t> &cu, int chunk) {
  std::vector<int32_t> index;
  std::vector<int4> items;
  if (p.mode == kPlanVarlenItems) {
    host_planner(p, cu, index, items);
    p.index = index.data();
    p.items = items.data();
  }
  p.cu = cu.data();
  p.order = nullptr;
  const int N = p.n_seq;
  int cnt = p.max_items;
  if (p.mode == kPlanVarlenDirect) cnt = N;
  if (p.mode == kPlanVarlenItems) cnt = index[0];
  EXPECT(cnt <= p.max_items || p.mode == kPlanVarlenDirect);
  int prev_last = 0;
  for (int n = 0; n < N; ++n) {
    int first = -1, last = -1;
    seq_items(p, n, first, last);
    EXPECT(first == prev_last && last > first && last <= cnt);
    prev_last = last;
    int t = cu[n];
    for (int i = first; i < last; ++i) {
      Item it;
      EXPECT(load_item(p, i, it));
      EXPECT(it.n == n && it.t0 == t && it.t1 >= it.t0 && it.t1 <= cu[n + 1]);
      EXPECT((it.t0 - cu[n]) % chunk == 0);  // chunks start at the sequence start
      if (p.mode != kPlanVarlenDirect) EXPECT(it.t1 - it.t0 <= p.seg_len);
      EXPECT(((it.flags & kFirstSeg) != 0) == (i == first));
      EXPECT(((it.flags & kLastSeg) != 0) == (i == last - 1));
      if (!(it.flags & kFirstSeg)) EXPECT(i - 1 >= 0 && i - 1 < p.max_items);
      if (!(it.flags & kLastSeg)) EXPECT(i + 1 < p.max_items);
      EXPECT(i < p.max_items || p.mode == kPlanVarlenDirect);
      // a segment that is not a sequence's last is never empty
      if (!(it.flags & kLastSeg)) EXPECT(it.t1 > it.t0);
      t = it.t1;
    }
    EXPECT(t == cu[n + 1]);
  }
  // every dispatch slot decodes to an item (identity order)
  for (int s = 0; s < cnt; ++s) {
    int idx = -1;
    Item it;
    EXPECT(slot_item(p, s, idx, it) && idx == s);
  }
  Item it;
  int idx;
  EXPECT(!slot_item(p, cnt, idx, it));
}

// One planned call: the item tiling, the workspace regions and the
// workgroup mappings its launches use.
void check_forward(const HostPlan &hp, const std::vector<int32_t> &cu, int H, int dk, int dv,
                   bool norm) {
  const Plan &p = hp.p;
  EXPECT(hp.chunk == 64 || hp.chunk == 32);
  EXPECT(hp.ndt >= 1 && dv % hp.ndt == 0);
  check_items(p, cu, hp.chunk);
  const long long units = (long long)p.max_items * H;
  check_mapping(p.mode == kPlanFixed ? 0 : 1, units, hp.ndt);  // output pass
  if (hp.segmented) check_mapping(1, units, hp.ndt);           // state pass
  const size_t slot_bytes = (size_t)p.max_items * H * dk * dv * sizeof(float);
  if (hp.segmented) {
    EXPECT(hp.off_slots % 256 == 0);
    const size_t slots_end = hp.off_slots + slot_bytes;
    if (norm) {
      EXPECT(hp.off_zslots >= slots_end && hp.off_zslots % 256 == 0);
      EXPECT(hp.off_zslots + (size_t)p.max_items * H * dk * sizeof(float) <= hp.ws_bytes);
    } else {
      EXPECT(slots_end <= hp.ws_bytes);
    }
  }
  if (p.mode == kPlanVarlenItems) {
    EXPECT(hp.off_index + sizeof(int32_t) * ((size_t)p.n_seq + 2) <= hp.off_items);
    EXPECT(hp.off_items + sizeof(int4) * (size_t)p.max_items <= hp.off_order);
  }
  if (hp.ordered) {
    EXPECT(p.max_items <= kOrderMaxItems || p.mode == kPlanVarlenDirect);
    const size_t n_order = p.mode == kPlanVarlenDirect ? (size_t)p.n_seq : (size_t)p.max_items;
    EXPECT(hp.off_order % 256 == 0 && hp.off_order + 4 * n_order <= hp.ws_bytes);
  }
  if (!hp.segmented && !hp.ordered) EXPECT(hp.ws_bytes == 0);
}

// The chained scan's workspace (local, inclusive and incoming states, then
// the flags, each 256-byte aligned, no overlap, nothing past the query's
// size) and its workgroup -> (head, d_v tile) dealing: a bijection within
// each item whose XCD (id mod 8) is the same for every d_v tile of a head.
void check_chain(const HostPlan &hp, int H, int dk, int dv) {
  const Plan &p = hp.p;
  EXPECT(hp.segmented && hp.fast && p.mode == kPlanFixed);
  EXPECT(fwd_chain_ok(dk, H, p.G));
  const size_t slot_bytes = (size_t)p.max_items * H * dk * dv * sizeof(float);
  EXPECT(hp.off_slots == 0 && hp.off_incl % 256 == 0 && hp.off_sin % 256 == 0 &&
         hp.off_flags % 256 == 0);
  EXPECT(hp.off_incl >= slot_bytes && hp.off_sin >= hp.off_incl + slot_bytes &&
         hp.off_flags >= hp.off_sin + slot_bytes);
  EXPECT(hp.off_flags + (size_t)p.max_items * H * hp.ndt * sizeof(int32_t) == hp.ws_bytes);
  const int U = H * hp.ndt;
  EXPECT(U % 8 == 0);
  std::vector<int> seen((size_t)U, 0), xcd_of_head((size_t)H, -1);
  for (int u = 0; u < U; ++u) {
    int h = -1, dt = -1;
    chain_unit(u, U, hp.ndt, h, dt);
    EXPECT(h >= 0 && h < H && dt >= 0 && dt < hp.ndt);
    if (h < 0 || h >= H || dt < 0 || dt >= hp.ndt) continue;
    ++seen[(size_t)h * hp.ndt + dt];
    if (xcd_of_head[h] < 0) xcd_of_head[h] = u & 7;
    EXPECT(xcd_of_head[h] == (u & 7));
  }
  for (int c : seen) EXPECT(c == 1);
}

void check_backward(const BwdPlan &bp, const std::vector<int32_t> &cu, int H, int dk, int dv,
                    long long total_T) {
  const HostPlan &hp = bp.hp;
  check_forward(hp, cu, H, dk, dv, false);
  if (bp.wide) {
    EXPECT(bp.ndt == 1 && bp.dvt == dv && bp.part_bytes == 0);
    check_mapping(hp.p.mode == kPlanFixed ? 0 : 1, (long long)hp.p.max_items * H, 1);
    // the fused launch (no segments) starts the dq walk at an id that is a
    // multiple of 8, so both walks keep the id -> XCD dealing
    EXPECT(xcd_grid(hp.p.mode == kPlanFixed ? 0 : 1, (long long)hp.p.max_items * H, 1) % 8 == 0);
  }
  if (total_T == 0) return;
  const size_t slot_bytes = (size_t)hp.p.max_items * H * dk * dv * sizeof(float);
  if (hp.segmented) EXPECT(bp.off_cslots + slot_bytes <= bp.off_part);
  // partial rows [d_v tile][H][token][dk] fp32 for dq, then for dk
  const size_t part = (size_t)bp.ndt * H * total_T * dk * sizeof(float);
  if (!bp.wide) EXPECT(bp.part_bytes >= part && bp.off_part + 2 * bp.part_bytes <= bp.ws_bytes);
  EXPECT(bp.ws_bytes >= bp.off_part);
}

void fixed_case(int dt, int B, int T, int H, int dk, int dv, int chunk, long long target) {
  set_target(target);
  char b[160];
  snprintf(b, sizeof b, "fixed dt%d B%d T%d H%d dk%d dv%d C%d target %lld", dt, B, T, H, dk, dv,
           chunk, target);
  where = b;
  std::vector<int> lens((size_t)B, T);
  const std::vector<int32_t> cu = cu_of(lens);
  const HostPlan hp = plan_fwd_fixed(dt, B, T, H, dk, dv, chunk);
  if (T > 0) check_forward(hp, cu, H, dk, dv, false);
  if (hp.chain) check_chain(hp, H, dk, dv);
  // the chained scan (when selected) takes every segmented bf16 matrix-core
  // plan it can
  EXPECT(hp.chain == (fwd_chain_enabled() && hp.fast && hp.segmented &&
                      fwd_chain_ok(dk, H, hp.p.G)));
  EXPECT(hp.ws_bytes == gla_chunk_fwd_workspace_bytes((gla_dtype)dt, B, T, H, dk, dv, chunk));
  const HostPlan hz = plan_linear_attn(dt, B, T, H, dk, dv, chunk);
  if (T > 0) check_forward(hz, cu, H, dk, dv, true);
  const BwdPlan bp =
      bwd_layout(bwd_plan_fixed(dt, B, T, H, dk, dv, chunk), (long long)B * T, H, dk, dv);
  if (T > 0) check_backward(bp, cu, H, dk, dv, (long long)B * T);
  EXPECT(bp.ws_bytes == gla_chunk_bwd_workspace_bytes((gla_dtype)dt, B, T, H, dk, dv, chunk));
}

void varlen_case(int dt, const std::vector<int> &lens, int H, int dk, int dv, int chunk,
                 long long target, bool noalloc_fits) {
  set_target(target);
  const std::vector<int32_t> cu = cu_of(lens);
  const int N = (int)lens.size();
  const int total = cu[N];
  char b[160];
  snprintf(b, sizeof b, "varlen dt%d N%d total %d H%d dk%d dv%d C%d target %lld", dt, N, total,
           H, dk, dv, chunk, target);
  where = b;
  HostPlan hp = plan_varlen(dt, N, total, H, dk, dv, chunk);
  check_forward(hp, cu, H, dk, dv, false);
  EXPECT(hp.ws_bytes ==
         gla_chunk_fwd_varlen_workspace_bytes((gla_dtype)dt, N, total, H, dk, dv, chunk));
  if (noalloc_fits) EXPECT(hp.ws_bytes <= (size_t)GLA_NOALLOC_SCRATCH_BYTES);
  check_forward(plan_linear_attn_varlen(dt, N, total, H, dk, dv, chunk), cu, H, dk, dv, true);
  const BwdPlan bp = bwd_layout(
      bwd_plan_varlen(dt, N, total, H, dk, dv, chunk), total, H, dk, dv);
  check_backward(bp, cu, H, dk, dv, total);
  EXPECT(bp.ws_bytes ==
         gla_chunk_bwd_varlen_workspace_bytes((gla_dtype)dt, N, total, H, dk, dv, chunk));
}

std::vector<int> parse_lengths(const char *s) {
  std::vector<int> v;
  while (*s) {
    char *end = nullptr;
    const long x = strtol(s, &end, 10);
    if (end == s) break;
    v.push_back((int)x);
    s = *end == ',' ? end + 1 : end;
  }
  return v;
}

}  // namespace

int main(int argc, char **argv) {
  const int BF = GLA_BF16, F32 = GLA_F32;
  const long long targets[] = {0, 1, 100000};
  // head shapes: the Laplace head, the other matrix-core shapes, the
  // vector-ALU path
  const int shapes[][3] = {{BF, 96, 192}, {BF, 64, 128}, {BF, 128, 256}, {BF, 96, 256},
                           {BF, 96, 64},  {F32, 32, 64}, {F32, 16, 32}};
  for (long long tg : targets) {
    // the named workloads' plans
    fixed_case(BF, 8, 2048, 16, 96, 192, 64, tg);   // Laplace-shaped prefill
    fixed_case(BF, 1, 65536, 16, 96, 192, 64, tg);  // long context
    fixed_case(F32, 1, 256, 2, 16, 32, 32, tg);     // tiny check
    // the chained scan's plans (heads a multiple of 8), up to and past its
    // 256 segments per sequence, with and without it selected
    for (const char *chain : {"1", "0"}) {
      setenv("GLA_FWD_CHAIN", chain, 1);
      for (int H : {8, 16, 24})
        for (int T : {1000, 4097, 25600, 38400, 65536})
          for (const auto &sh : {std::array<int, 2>{96, 192}, std::array<int, 2>{96, 64},
                                 std::array<int, 2>{64, 128}})
            fixed_case(BF, 1 + (T < 5000), T, H, sh[0], sh[1], 0, tg);
    }
    unsetenv("GLA_FWD_CHAIN");
    for (const auto &sh : shapes)
      for (int T : {1, 63, 64, 65, 129, 1000, 4097})
        for (int chunk : {0, 32}) fixed_case(sh[0], 2, T, 3, sh[1], sh[2], chunk, tg);
    const std::vector<std::vector<int>> ragged = {
        {5, 0, 130, 1, 64, 65, 300}, {2000, 1, 700}, {0}, {1}, {0, 0, 0}, {65536},
        {9000, 3000},                {7000, 1, 5000}, {128, 129, 127}};
    for (const auto &l : ragged)
      for (const auto &sh : shapes) varlen_case(sh[0], l, 16, sh[1], sh[2], 0, tg, tg == 0);
    // the allocation-free entry point's largest default plans: 1 to 7 long
    // sequences at the Laplace head shape
    for (int n = 1; n <= 7; ++n)
      varlen_case(BF, std::vector<int>((size_t)n, 65536), 16, 96, 192, 0, tg, tg == 0);
    for (int i = 1; i < argc; ++i) {
      const std::vector<int> l = parse_lengths(argv[i]);
      for (const auto &sh : shapes) varlen_case(sh[0], l, 16, sh[1], sh[2], 0, tg, tg == 0);
    }
  }
  printf("plan_check: %lld checks, %d failures\n", checks, failures);
  return failures == 0 ? 0 : 1;
}
