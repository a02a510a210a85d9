// moe_plan.h -- host-side problem validation, tile choice and workspace layout.
//
// Pure C++ (no HIP calls), so it also builds with g++ for CPU tests.  The tile choice
// is an M-bucket table in the spirit of the per-M tile tables of the vLLM fused-MoE
// config page (section 03: one tile setting per bucket of the step's token count M),
// keyed here by the mean rows per routed expert, T*k/E.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "moe.h"
#include "moe_tuned.h"

namespace moe {
// internal linkage: every translation unit that includes this header gets its own copy, so
// two objects built with different settings can never exchange definitions at link time
namespace {

constexpr int kThreads = 256;          // threads per workgroup (4 wave64)
constexpr int kWaves = 4;
constexpr int kSlotInts = 1024;        // control slots sit 4 KB apart (separate HBM channels)
constexpr int kCtrlSlots = 48;
constexpr int kCtrlBytes = kCtrlSlots * kSlotInts * 4;  // control block at the start of the workspace
constexpr int kTicketParts = 8;        // ticket counters (see C_PTICKET)
constexpr int kXcds = 8;               // XCDs of the GPU: one late-phase ticket counter each (C_LTICKET)
constexpr int kGroupM = 4;             // late phase: m-tiles per group of the grouped item order
constexpr int kMaxE = 1024;
constexpr int kMaxFp8ScaleBlocks = 128;  // fp8: 128-wide scale blocks along one wave's K range
constexpr int kMaxK = 256;
constexpr int kTopkTokens = 16;        // tokens per top-k item (4 per wave)
constexpr int kTopkTokensSmall = 4;    // ... when all tokens form one scatter chunk (1 per wave)
// most parts the router's K is split into: 8 on the tile core (mg > 1) except in the fp8
// kernels, whose registers have no room for the top-k items to load 8 parts at once
constexpr int kMaxRouterSplit(bool fp8, int mg) { return (mg == 1 || fp8) ? 4 : 8; }

// router tiles on the tile core (mg > 1): 16-token groups per tile; 4 (64 tokens x 256
// experts) only in the 128- and 160-row kernels, whose registers hold it without spilling,
// else 1 (16 tokens x 128 experts)
constexpr int router_groups(int mg) { return mg >= 8 ? 4 : 1; }
constexpr int kMaxChunkTokens = 128;   // tokens per scatter chunk (rank bitmasks: 4 words)
constexpr int kMaxChunkSlots = 1024;   // (token, slot) pairs per chunk
constexpr int kCombineUnroll = 2;      // combine: (token, column) pairs per thread in flight
constexpr int kMaxCombineTokens = 4;   // tokens per combine item (Tiles::ctok) at most
constexpr int kMaxCombineSlots = kMaxCombineTokens * kMaxK;  // (token, slot) pairs per combine item
constexpr int kZeroPerItem = 2048;     // dependency counters cleared per zeroing item
constexpr int kQuantTokens = 16;       // tokens per activation-quantisation item (fp8 activations)


// control-block slots (one int32 each, at int index slot * kSlotInts): a poll of one
// counter never shares a cache line or channel with the ticket counter or another counter.
// C_PTICKET + p (p < kTicketParts): ticket counter of partition p; C_LTICKET + x (x < kXcds):
// late-phase ticket counter of XCD x; see the persistent kernel.  Slots not named here are
// unused.
enum CtrlSlot : int {
  C_MAGIC = 0, C_ZDONE = 2, C_LDONE = 3, C_KDONE = 4, C_SDONE = 6, C_EXIT = 8, C_ERR = 10, C_QDONE = 12,
  C_PTICKET = 16, C_PLANB = 24, C_LTICKET = 32, C_NSLOTS = kCtrlSlots
};
// C_PLANB .. C_PLANB + 7: copies of the plan flag (n_mt + 1 once the plan is published),
// eight per slot, 512 bytes apart; workgroup b polls copy b % kPlanCopies
constexpr int kPlanCopies = 64;
constexpr int plan_flag_word(int c) { return kSlotInts * (C_PLANB + (c >> 3)) + (c & 7) * 128; }
constexpr int kMagic = 0x4d6f4531;     // "MoE1"

// which phases a launch runs
enum PhaseBits : int { PH_ROUTE = 1, PH_PERMUTE = 2, PH_FFN = 4, PH_COMBINE = 8, PH_IDS_GIVEN = 16 };

struct Tiles {
  int mg;          // 16-row token groups per m-tile (1, 2, 4, 8 or 10)
  int bm;          // rows per m-tile = 16 * mg
  int nf;          // 16-row weight fragments per wave (2 when mg == 1, else 4)
  int gu_cols;     // H columns per gate/up item: 4 waves x nf/2 x 16 (16 when mg == 1)
  int dn_cols;     // output columns per down item: 4 waves x nf x 16 (128 when mg == 1)
  int tk;          // tokens per scatter chunk (tk <= 128, tk * k <= 1024)
  int ctok;        // tokens per combine item (1 for small T: more items in parallel)
  int rt_tokens;   // router item: tokens x experts (16 x 16 split over the 4 waves when
  int rt_experts;  //   mg == 1, else 16 * router_groups(mg) x 64 * NF on the expert tile core)
  int rt_split;    // K splits per router tile (1, 2, 4 or 8): with few tiles, each item takes
                   //   one part of K and the top-k items add the partial sums in order
  int late;        // 1: gate/up and down items come from per-XCD queues in grouped order
                   //   (m-tiles of more than 16 rows, dynamic schedule), see the kernel
  int group_m;     // late phase: m-tiles per group (items of a group run n-tile-major)
  int aq;          // 1: the expert GEMMs read fp8 activations (MOE_AQ_FP8, m-tiles above 16 rows)
};

struct Layout {
  Tiles tiles;
  int64_t T;
  int E;
  int n_lt, n_le;        // router items: token tiles x expert blocks
  int n_kt;              // top-k items (kt_tok tokens each)
  int kt_tok;            // tokens per top-k item: kTopkTokensSmall when n_kc == 1, else kTopkTokens
  int n_kc;              // scatter chunks
  int mt_routed_max;     // bound on routed m-tiles
  int n_shmt;            // shared-expert m-tiles
  int nt_gu, nt_dn;      // gate/up and down items per m-tile
  int n_comb;            // combine items
  int64_t rows_h;        // rows of H and Y: T*k + n_shared*T
  int xs_stride, hs_stride;  // fp8 activations: bytes per row of the hidden / H block scales
  // byte offsets into the workspace
  size_t off_gudone, off_desc, off_logits, off_lpart, off_ids, off_wts, off_hist, off_counts, off_offsets, off_mtoff,
      off_perm, off_invperm, off_mtok, off_slotmt, off_xq, off_xs, off_hs, off_h, off_y, total;
};

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

inline size_t dtype_size(int dt) { return dt == MOE_F32 ? 4 : (dt == MOE_BF16 ? 2 : 1); }

// Checks shapes and dtypes only (no pointers).
inline moe_status validate_problem(const moe_problem *p) {
  if (!p) return MOE_ERR_INVALID_ARGUMENT;
  if (p->T < 0 || p->d <= 0 || p->n <= 0 || p->E <= 0 || p->k <= 0) return MOE_ERR_INVALID_ARGUMENT;
  if (p->k > p->E) return MOE_ERR_INVALID_ARGUMENT;
  if (p->n_shared != 0 && p->n_shared != 1) return MOE_ERR_INVALID_ARGUMENT;
  const int a = p->act_dtype, w = p->w_dtype;
  if (a < 0 || a > 2 || w < 0 || w > 2) return MOE_ERR_INVALID_ARGUMENT;
  const bool ok = (a == MOE_F32 && w == MOE_F32) || (a == MOE_BF16 && w == MOE_BF16) ||
                  (a == MOE_BF16 && w == MOE_FP8_E4M3);
  if (!ok) return MOE_ERR_UNSUPPORTED;
  if (w == MOE_FP8_E4M3) {
    if (p->scale_block != 128) return MOE_ERR_UNSUPPORTED;
    // a wave of the 16-row units keeps the block scales of its K range in two lane registers
    // (128 blocks of 128): gate/up units take half of d, down units all of n
    if (p->d > kMaxFp8ScaleBlocks * 2 * 128 || p->n > kMaxFp8ScaleBlocks * 128) return MOE_ERR_UNSUPPORTED;
  } else if (p->scale_block != 0) {
    return MOE_ERR_INVALID_ARGUMENT;
  }
  if (p->w_layout != MOE_W_ROWMAJOR && p->w_layout != MOE_W_PACKED) return MOE_ERR_INVALID_ARGUMENT;
  if (p->act_quant != MOE_AQ_NONE && p->act_quant != MOE_AQ_FP8) return MOE_ERR_INVALID_ARGUMENT;
  if (p->act_quant == MOE_AQ_FP8 && w != MOE_FP8_E4M3) return MOE_ERR_UNSUPPORTED;
  if (p->E > kMaxE || p->k > kMaxK) return MOE_ERR_UNSUPPORTED;
  if (p->d % 256 || p->n % 256) return MOE_ERR_UNSUPPORTED;
  if (p->T * (int64_t)p->k >= (int64_t(1) << 31) - 1) return MOE_ERR_UNSUPPORTED;
  if (p->T * (int64_t)(p->d > p->n ? p->d : p->n) >= (int64_t(1) << 40)) return MOE_ERR_UNSUPPORTED;
  // the tile core addresses activation rows (hidden, H) with 32-bit offsets
  const int64_t asz = a == MOE_F32 ? 4 : 2, rows_h = p->T * (int64_t)p->k + (int64_t)p->n_shared * p->T;
  if (p->T * (int64_t)p->d * asz >= (int64_t(1) << 32) || rows_h * (int64_t)p->n * asz >= (int64_t(1) << 32))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// the tile of a given m-tile size (mg 16-row groups) and late-phase group size
inline Tiles tiles_for(const moe_problem *p, int mg, int group_m) {
  Tiles t;
  t.mg = mg;
  t.bm = 16 * t.mg;
  t.nf = t.mg == 1 ? 2 : 4;
  // mg == 1: small units streamed by single waves (gate/up: 16 columns, the waves split
  // gate/up and the two halves of K; down: 32 channels per wave)
  t.gu_cols = t.mg == 1 ? 16 : 4 * (t.nf / 2) * 16;
  t.dn_cols = t.mg == 1 ? 128 : 4 * t.nf * 16;
  t.tk = kMaxChunkSlots / p->k;
  if (t.tk > kMaxChunkTokens) t.tk = kMaxChunkTokens;
  if (t.tk < 1) t.tk = 1;
  t.ctok = p->T > 1024 ? kMaxCombineTokens : 1;
  t.late = t.mg > 1 ? 1 : 0;
  t.group_m = group_m;
  t.aq = (p->act_quant == MOE_AQ_FP8 && t.mg > 1) ? 1 : 0;
  t.rt_tokens = t.mg == 1 ? 16 : 16 * router_groups(t.mg);
  t.rt_experts = t.mg == 1 ? 16 : router_groups(t.mg) == 1 ? 128 : 256;
  return t;
}

// The tile from the M-bucket table (moe_tuned.h), keyed by the mean rows per routed expert.
// The row count of an expert spreads around the mean by about its square root, so a bucket's
// m-tile is chosen for most experts to fit in one m-tile (each extra m-tile re-reads the
// expert's weights).  Rule lists: f32, bf16, fp8 weights, fp8 weights with fp8 activations.
inline int tile_table_row(const moe_problem *p) {
  if (p->w_dtype == MOE_F32) return 0;
  if (p->w_dtype == MOE_BF16) return 1;
  return p->act_quant == MOE_AQ_FP8 ? 3 : 2;
}

inline Tiles choose_tiles(const moe_problem *p) {
  const double mean_rows = p->E > 0 ? double(p->T) * p->k / p->E : 0.0;
  const int wd = tile_table_row(p);
  const TileRule *rule = &kTileRules[wd][kNumTileRules - 1];
  for (int i = 0; i < kNumTileRules; ++i)
    if (mean_rows <= kTileRules[wd][i].max_mean_rows) {
      rule = &kTileRules[wd][i];
      break;
    }
  return tiles_for(p, rule->m_tile_rows / 16, rule->group_m);
}

// An m-tile size and group size given by the caller (0: the table's); false if not valid
inline bool override_tiles(const moe_problem *p, int m_tile_rows, int group_m, Tiles *t) {
  *t = choose_tiles(p);
  if (group_m < 0 || group_m > 64) return false;
  if (m_tile_rows != 0) {
    const int r = m_tile_rows;
    if (r != 16 && r != 32 && r != 64 && r != 128 && r != 160) return false;
    *t = tiles_for(p, r / 16, t->group_m);
  }
  if (group_m != 0) t->group_m = group_m;
  return true;
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// words of one per-m-tile counter array (gate/up done, down done), padded to 256 bytes
inline int ctr_words(const Layout &L) { return (int)align_up((size_t)(L.mt_routed_max + L.n_shmt + 1), 64); }

// Work items of one launch, per phase, in order: Z (clear counters), L (router), K (top-k),
// SG (shared gate/up), Q (fp8 activations: quantise the hidden rows), S (scatter); the
// routed gate/up, down and combine items follow and are counted on the device once the plan
// exists.  The Z and router items take no ticket (each workgroup runs its share of them
// first); the others are handed out by ticket in this order.
struct PhaseCounts {
  int gd_words, hist_words;  // words cleared by Z items: dependency counters, chunk histograms
  int z, l, k, sg, s;
  int q;                     // activation-quantisation items (fp8 activations; ticketed before S)
};

inline Layout make_layout(const moe_problem *p, const Tiles *forced = nullptr) {
  Layout L{};
  L.tiles = forced ? *forced : choose_tiles(p);
  const int64_t T = p->T, k = p->k, E = p->E, bm = L.tiles.bm;
  L.T = T;
  L.E = (int)E;
  L.n_lt = (int)ceil_div(T, L.tiles.rt_tokens);
  L.n_le = (int)ceil_div(E, L.tiles.rt_experts);
  // a router item's waves each issue one chunk of loads (16 steps, 512 K) per memory round
  // trip, and one item's loads are bounded by its CU's bandwidth: with few tiles and K above
  // 1024, K is split over 2 or 4 items per tile (each wave's part of K stays a multiple of
  // 32; the top-k items add the parts, one 16-byte load each).  Short K is not split: the
  // router items are the first of the launch, and more of them only start later.
  // Tile-core router items (mg > 1) split K until there are 256 items or 8 parts; each part
  // stays a multiple of 128, the longest K chunk of the tile core.
  L.tiles.rt_split = 1;
  if (L.tiles.mg == 1 && (int64_t)L.n_lt * L.n_le < 64 && p->d > 1024)
    L.tiles.rt_split = (p->d > 4096 && p->d % 512 == 0) ? 4 : 2;
  if (L.tiles.mg > 1)
    while (L.tiles.rt_split < kMaxRouterSplit(p->w_dtype == MOE_FP8_E4M3, L.tiles.mg) &&
           (int64_t)L.n_lt * L.n_le * L.tiles.rt_split < 256 &&
           p->d % (256 * L.tiles.rt_split) == 0)
      L.tiles.rt_split *= 2;
  L.n_kc = (int)ceil_div(T, L.tiles.tk);
  // one scatter chunk: the top-k items take a token per wave (the selection rounds of
  // several tokens per wave cost more than the extra items), and the last of them plans and
  // scatters every token; else 16 tokens per item, chunk histograms and scatter items
  L.kt_tok = L.n_kc <= 1 ? kTopkTokensSmall : kTopkTokens;
  L.n_kt = (int)ceil_div(T, L.kt_tok);
  const int64_t tk = T * k;
  int64_t bound = tk / bm + (E < tk ? E : tk);
  if (bound > tk) bound = tk;
  L.mt_routed_max = (int)bound;
  L.n_shmt = p->n_shared ? (int)ceil_div(T, bm) : 0;
  L.nt_gu = p->n / L.tiles.gu_cols;
  L.nt_dn = (int)ceil_div(p->d, L.tiles.dn_cols);
  L.n_comb = (int)ceil_div(T, L.tiles.ctok);
  L.rows_h = tk + (int64_t)p->n_shared * T;
  // fp8 activations: one scale byte per 128-wide block, rows padded to whole dwords
  L.xs_stride = (int)align_up((size_t)(p->d / 128), 4);
  L.hs_stride = (int)align_up((size_t)(p->n / 128), 4);
  const size_t asz = dtype_size(p->act_dtype), hsz = L.tiles.aq ? 1 : asz;
  const bool aq = L.tiles.aq != 0;
  size_t o = kCtrlBytes;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  // per m-tile counters: gate/up items done, then (from word ctr_words) down items done; the
  // two arrays start on separate 256-byte lines, so the down items' atomics never share a
  // line with the gate/up counters that down units poll
  L.off_gudone = take(sizeof(int32_t) * 2 * (size_t)ctr_words(L));
  L.off_desc = take(4 * sizeof(int32_t) * (size_t)(L.mt_routed_max + 1));
  L.off_logits = take(sizeof(float) * (size_t)(T * E));
  L.off_lpart = take(L.tiles.rt_split > 1 ? sizeof(float) * (size_t)L.tiles.rt_split * (size_t)(T * E) : 0);
  L.off_ids = take(sizeof(int32_t) * (size_t)tk);
  L.off_wts = take(sizeof(float) * (size_t)tk);
  L.off_hist = take(sizeof(int32_t) * (size_t)L.n_kc * (size_t)E);
  L.off_counts = take(sizeof(int32_t) * (size_t)E);
  L.off_offsets = take(sizeof(int32_t) * (size_t)(E + 1));
  L.off_mtoff = take(sizeof(int32_t) * (size_t)(E + 1));
  L.off_perm = take(sizeof(int32_t) * (size_t)tk);
  L.off_invperm = take(sizeof(int32_t) * (size_t)tk);
  L.off_mtok = take(sizeof(int32_t) * (bm == 16 ? (size_t)L.mt_routed_max * 16 : 16));
  L.off_slotmt = take(sizeof(int32_t) * (size_t)tk);
  L.off_xq = take(aq ? (size_t)T * (size_t)p->d : 0);
  L.off_xs = take(aq ? (size_t)T * (size_t)L.xs_stride : 0);
  L.off_hs = take(aq ? (size_t)L.rows_h * (size_t)L.hs_stride : 0);
  L.off_h = take(hsz * (size_t)L.rows_h * (size_t)p->n);
  L.off_y = take(asz * (size_t)L.rows_h * (size_t)p->d);
  L.total = o;
  return L;
}

// late: the launch takes its gate/up and down items from the per-XCD queues (Tiles::late and
// the dynamic schedule)
inline PhaseCounts phase_counts(const Layout &L, int phases, bool late) {
  PhaseCounts c{};
  const bool ffn = (phases & PH_FFN) != 0, perm = (phases & PH_PERMUTE) != 0;
  const bool many = L.n_kc > 1;  // else the last top-k item plans and scatters by itself
  c.gd_words = ffn ? 2 * ctr_words(L) : 0;
  c.hist_words = (perm && many) ? L.n_kc * L.E : 0;
  c.z = (int)ceil_div(c.gd_words + c.hist_words, kZeroPerItem);
  c.l = (phases & PH_ROUTE) ? L.n_lt * L.n_le * L.tiles.rt_split : 0;
  c.k = (phases & (PH_ROUTE | PH_PERMUTE)) ? L.n_kt : 0;
  // (with the late phase, the shared expert's gate/up items are late items too)
  c.sg = (ffn && !late) ? L.n_shmt * L.nt_gu : 0;
  c.s = (perm && many) ? L.n_kc : 0;
  c.q = (ffn && L.tiles.aq) ? (int)ceil_div(L.T, kQuantTokens) : 0;
  return c;
}

}  // namespace
}  // namespace moe
