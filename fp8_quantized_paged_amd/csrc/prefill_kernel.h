// Chunked causal prefill attention over an FP8 (e4m3) paged cache on FP8 matrix
// cores (gfx950 v_mfma_f32_32x32x64_f8f6f4).
//
// Method: "vLLM FP8 KV-Cache and Attention Quantization Update" (agentlenshq.com):
// queries and softmax probabilities are quantised to FP8 so both attention
// contractions run on FP8 tensor instructions (introduction and section "Kernel
// and fusion optimizations"), with partial sums flushed to true float32 registers
// every chunk (section "Two-level accumulation"); head_dim 256 prefill is the case
// the pages single out (section "Per-architecture results").
//
// Formulation.  Both products are computed transposed, so that the score tile
// leaves the first MFMA in exactly the register layout the second MFMA takes as
// its B operand (no shuffle between them):
//   S^T[key][row]  = K[key][:] . Qc^T[:][row]          (A = K from LDS, B = Q codes)
//   O^T[dim][row] += V^T[dim][key] . P'^T[key][row]    (A = V^T from LDS, B = P')
// A "row" is one (query position, query head) pair; the G query heads of a KV head
// are stacked as rows, so one K/V tile serves the whole GQA group.  The 64-key
// contraction of the second product visits keys in a permuted order (the order in
// which the score lanes hold them); V^T is laid out in LDS in that same order.
//
// Work split.  A workgroup (4 waves) owns 128 rows of one (sequence, KV head) and
// streams that head's keys in 64-key tiles (4 pages) through double-buffered LDS;
// each wave owns 32 rows.  Workgroups are numbered KV-head-fastest so that, with
// the hardware's round-robin placement over the 8 XCDs, each XCD's L2 serves the
// keys of one KV head (when the KV head count divides 8).
//
// Softmax.  float32 online softmax in the log2 domain with a lazily moved
// reference: when a row's scores pass the reference by more than 8 log2 units (or at
// its first visible key) the reference is reset to the row's maximum minus kRefTop,
// so the weights p stay <= 2^8 and the largest weight seen sits at 2^kRefTop (2^4),
// well inside the e4m3 range.  (A reference at the maximum itself would leave the
// e4m3 range below 1 only 2^-9..1: after one dominant key, every ordinary key of a
// long row -- e.g. 11 log2 units lower -- would round to zero.)  2^4 rather than
// 2^6 leaves 4 log2 units of headroom, so rows reset rarely (head_dim-256 workload:
// 1525 us at 2^4, 1553 us at 2^5, 1598 us at 2^6, same box, round-robin).
// P' = e4m3(p * v_scale_j / (v_ref * prob_scale)), where v_ref is a running maximum of the per-token V scales (per-token-head mode) or
// the per-tensor V scale; folding v_scale_j into P' before rounding lets the FP8
// product carry per-token V scales.  The row sum l accumulates the same rounded
// P' (mapped back by v_ref * prob_scale / v_scale_j), so the output stays a convex
// combination of V rows.
//
// Accumulation (the pages' two-level scheme).  Level 1 is one MFMA's 64-key (PV) or
// 64-dim (QK) sum inside the matrix core, whose internal alignment is coarser than
// float32.  Level 2, the running output, is float32 in one of two forms (template
// flag kValuAdd, selectable per call): the MFMA's own float32 C operand, into which
// each 64-key chunk is added (the default), or a zeroed accumulator per chunk added
// into the output by float32 vector adds (the pages' explicit flush).  On gfx950 the
// two agree at 131,072 keys (tests/test_gpu_prefill.py, long-context planted-key
// test), i.e. the C operand is a true float32 accumulator.
#pragma once

#include "kvq_device.h"
#include "kvq_host.h"

namespace kvq {
namespace pf {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kRows = 32;                 // rows per wave
constexpr int kWgRows = kWaves * kRows;   // rows per workgroup
constexpr int kTile = 64;                 // keys per tile (4 pages)
constexpr int kTilePages = kTile / kPage;
constexpr float kSlack = 8.0f;            // log2 units: p <= 2^8
constexpr float kRefTop = 4.0f;           // log2 units: a reset puts the row maximum here
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kE4m3Max = 448.0f;

__device__ __forceinline__ v16f mfma(v8i a, v8i b, v16f c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// d[e] = p[e] * (f of lane r0 + e of this lane's 16-lane row), e = 0..3: v_mul_f32 with
// the DPP row_newbcast source operand, so the broadcast costs no instruction.  The
// leading s_nop covers the two wait states a DPP read needs after a vector write of
// its source register.
__device__ __forceinline__ void mul4_row_bcast(float (&d)[4], float f, int r0,
                                               const float (&p)[4]) {
#define KVQ_MUL4(R0)                                                                     \
  case R0:                                                                              \
    asm("s_nop 1\n\t"                                                                   \
        "v_mul_f32_dpp %0, %4, %5 row_newbcast:" #R0 " row_mask:0xf bank_mask:0xf\n\t"    \
        "v_mul_f32_dpp %1, %4, %6 row_newbcast:%9 row_mask:0xf bank_mask:0xf\n\t"         \
        "v_mul_f32_dpp %2, %4, %7 row_newbcast:%10 row_mask:0xf bank_mask:0xf\n\t"        \
        "v_mul_f32_dpp %3, %4, %8 row_newbcast:%11 row_mask:0xf bank_mask:0xf"              \
        : "=&v"(d[0]), "=&v"(d[1]), "=&v"(d[2]), "=&v"(d[3])                              \
        : "v"(f), "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]), "n"(R0 + 1), "n"(R0 + 2),  \
          "n"(R0 + 3));                                                                 \
    break
  switch (r0) {
    KVQ_MUL4(0); KVQ_MUL4(4); KVQ_MUL4(8); default: KVQ_MUL4(12);
  }
#undef KVQ_MUL4
}
// acc += d[e] * (f of lane r0 + e of this lane's row), e = 0..3, as four v_fmac_f32 with
// the DPP row_newbcast source (the compiler does not fold DPP into v_fmac).  The
// leading s_nop covers the two wait states a DPP read needs after a vector write of
// its source register.
__device__ __forceinline__ void fmac4_row_bcast(float& acc, float f, int r0, float d0, float d1,
                                                float d2, float d3) {
#define KVQ_FMAC4(R0)                                                                       \
  case R0:                                                                                 \
    asm volatile("s_nop 1\n\t"                                                             \
                 "v_fmac_f32_dpp %0, %1, %2 row_newbcast:" #R0 " row_mask:0xf bank_mask:0xf\n\t" \
                 "v_fmac_f32_dpp %0, %1, %3 row_newbcast:%6 row_mask:0xf bank_mask:0xf\n\t"      \
                 "v_fmac_f32_dpp %0, %1, %4 row_newbcast:%7 row_mask:0xf bank_mask:0xf\n\t"      \
                 "v_fmac_f32_dpp %0, %1, %5 row_newbcast:%8 row_mask:0xf bank_mask:0xf"            \
                 : "+v"(acc)                                                               \
                 : "v"(f), "v"(d0), "v"(d1), "v"(d2), "v"(d3), "n"(R0 + 1), "n"(R0 + 2),   \
                   "n"(R0 + 3));                                                           \
    break
  switch (r0) {
    KVQ_FMAC4(0); KVQ_FMAC4(4); KVQ_FMAC4(8); default: KVQ_FMAC4(12);
  }
#undef KVQ_FMAC4
}

// Key order inside a 64-key tile.  The A operand of S^T = K . Q^T is loaded so that
// MFMA row i (0..63) holds key tile_key(i) = 32 (i / 32) + 16 ((i / 4) % 2)
// + 4 ((i % 32) / 8) + i % 4.  With the 32x32 result layout (lane l, register r of
// key block kb holds row i = 32 kb + 8 (r / 4) + 4 (l / 32) + r % 4) this puts, in
// lane group gg = l / 32, register r of key block kb on key 32 kb + 16 gg + r: page
// 2 kb + gg, token r.  So the P' bytes a lane packs in register order are whole
// pages, and the matching V^T operand bytes are whole 16-token rows of the
// dim-major V tiles, which the loads copy unchanged.
__device__ __forceinline__ int tile_key(int i) {
  const int j = i % 32;
  return 32 * (i / 32) + 16 * ((j / 4) % 2) + 4 * (j / 8) + j % 4;
}

// Pipeline.  K (with the per-token scales) and V travel in separate LDS rings: the K
// operand of tile t + 1 is read one tile before the V operand of tile t + 1, so each
// ring is refilled as soon as its own contents are dead.  Iteration t runs phase 1
// (S^T of tile t + 1, P' of tile t), one workgroup barrier, then phase 2 (P.V of tile
// t, row sum and scaled scores).  The barrier of iteration t publishes K of tile t + 2
// and V of tile t + 1.  Phase 1 issues the loads of K of tile t + 3 (its slot held K of
// tile t - 1, last read before the previous barrier) and of V of tile t + 2 (its slot
// held V of tile t - 2, likewise), so each load has one and a half iterations to land,
// and the operand reads of phase 2's first chunks are issued before the barrier.
constexpr int kKSlots = 4;  // power-of-two rings: slot = tile index & 3
constexpr int kVSlots = 4;
constexpr int kFSlots = 2;  // per-wave factor blocks: tiles t and t + 1
// Block-table entries are fetched into LDS by direct loads, kIdTiles tiles' worth at a
// time, one chunk ahead of use.  (Reading them with vector loads inside the tile loop
// would put them in the same in-order completion count as the tile loads and force
// a wait for every tile in flight.)
constexpr int kIdTiles = 64;
static_assert(kIdTiles * kTilePages == kThreads, "one page id per thread per chunk");

// LDS layout.  Every tile region is an array of 16-byte chunks written by direct
// global->LDS loads: one load instruction writes 64 consecutive chunks, one per lane.
// Each load instruction reads from a single page, so its global address is that
// page's base (scalar registers) plus a per-lane offset that does not change from
// tile to tile.
//   K slot: page p (tile keys 16 p .. 16 p + 15) at chunks p * KPC + [0, 16 NC);
//       token t, dim chunk c (bytes 16 c .. 16 c + 15) at NC t + 2 ((c / 2) ^ phi(t))
//       + c % 2.  The XOR on 32-byte pairs and the odd page stride KPC = 16 NC + 1 put
//       the 16 rows one operand read touches (8 tokens of 2 pages, one chunk each) on
//       16 different bank groups.  Then KS, VS: the 64 keys' K and V scales
//       (per-token-head mode).
//   V slot: page p, channel d at chunk p * D + d: the page's 16 tokens of that channel.
//   Factor block (per wave, per tile): per-key factors derived from KS/VS: CF, the
//       score multiplier k_scale * q_scale * softmax_scale * log2(e); FV, the P'
//       factor v_scale / (v_ref * prob_scale); IF, its reciprocal.
template <int D>
struct Layout {
  static constexpr int NC = D / 16;            // 16-byte chunks per key row
  static constexpr int KPC = 16 * NC + 1;      // chunk stride of K pages
  static constexpr int K_CHUNKS = kTilePages * KPC;
  static constexpr int KS_OFF = 16 * K_CHUNKS;
  static constexpr int VS_OFF = KS_OFF + kTile * 4;
  static constexpr int K_BYTES = VS_OFF + kTile * 4;
  static constexpr int VT_CHUNKS = kTilePages * D;
  static constexpr int V_BYTES = 16 * VT_CHUNKS;
  static constexpr int CF_OFF = 0;
  static constexpr int FV_OFF = CF_OFF + kTile * 4;
  static constexpr int IF_OFF = FV_OFF + kTile * 4;
  static constexpr int F_BYTES = IF_OFF + kTile * 4;
  // load instructions per page for K and for V (64 chunks each), and per wave per
  // tile for each
  static constexpr int PI = 16 * NC / kWave;
  static constexpr int W = kTilePages * PI / kWaves;
  static_assert(16 * NC == D && D % kWave == 0 && W >= 1, "head_dim");
  static_assert(kWaves % PI == 0, "instruction split");
  // pair swizzle of token t (keeps a 32-byte pair contiguous)
  static __device__ __forceinline__ int phi(int t) { return (t / (16 / NC)) % (NC / 2); }
};

struct PrefillArgs {
  const uint16_t* q;
  const int32_t* cu_q_lens;
  int32_t num_kv_heads, tiles;
  const int32_t* block_table;
  int32_t bt_stride;
  const int32_t* seq_lens;
  const uint8_t* k_pages;
  const uint8_t* v_pages;
  const float* k_scales;  // per-token-head pools [P][Hkv][16], or per-KV-head [Hkv]
  const float* v_scales;
  float q_scale, k_scale, v_scale, prob_scale, sm_log2;  // per-tensor K/V scales
  int32_t head_scales;   // k_scales / v_scales are per-KV-head arrays
  int32_t causal, window;
  void* out;
  int32_t out_f32;
  // Key splits (1: none).  With more, workgroup (x, split y) covers its share
  // [y T / nsplit, (y + 1) T / nsplit) of its sequence's T key tiles and writes the
  // unnormalised partial result of each of its kWgRows rows to the workspace (row
  // index (y gridDim.x + x) kWgRows + row); prefill_merge_kernel combines them.
  int32_t nsplit;
  float* ws_o;   // per row: O v_ref s, D floats (s = prob_scale per-token-head, else 1)
  float* ws_ml;  // per row: reference maximum m (log2 units) and row sum, two floats
};

template <typename T>
__device__ __forceinline__ T lds_read(const uint8_t* base, int byte_off) {
  return *reinterpret_cast<const T*>(base + byte_off);
}

// Two waves per SIMD (two workgroups per CU), so one wave's vector work overlaps the
// other's matrix work, where it fits: <= 256 registers per lane and <= 80 KB of LDS
// per workgroup.  head_dim 128, and head_dim 64 per-token-head, read the per-key
// factors (P' scale, its reciprocal, the K-scale score factor) from LDS at the
// instruction that uses them instead of queueing them in registers one chunk ahead
// with the operands (the queue cost 16-32 registers, which spilled ~50 at head_dim 64
// per-token-head).  head_dim 256 cannot (its accumulators alone take 128 registers);
// head_dim 64 per-tensor measured 2% slower at two waves.
template <int D, bool kPTH>
constexpr int prefill_waves_per_simd() { return D == 128 || (D == 64 && kPTH) ? 2 : 1; }

template <int D, int G, bool kPTH, bool kValuAdd>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(
    prefill_waves_per_simd<D, kPTH>()))) void prefill_kernel(const PrefillArgs a) {
  constexpr bool kLateFactors = prefill_waves_per_simd<D, kPTH>() == 2;  // read at use
  using LY = Layout<D>;
  constexpr int NP = kWgRows / G;  // query positions per workgroup
  constexpr int KS = D / 64;       // 64-dim steps of the QK contraction
  constexpr int DB = D / 32;       // 32-dim blocks of the output
  constexpr int PER_K = LY::W + (kPTH ? 1 : 0);  // K-side loads per wave per tile
  constexpr int PER_V = LY::W;                    // V-side loads per wave per tile
  __shared__ __align__(16) uint8_t k_lds[kKSlots][LY::K_BYTES];
  __shared__ __align__(16) uint8_t v_lds[kVSlots][LY::V_BYTES];
  __shared__ __align__(16) uint8_t f_lds[kWaves][kFSlots][LY::F_BYTES];
  // physical page ids of the workgroup's tiles, kIdTiles tiles per chunk, two chunks
  __shared__ __align__(16) int ids_lds[2][kIdTiles * kTilePages];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int hkv = a.num_kv_heads;
  const int g = (int)(blockIdx.x % (unsigned)hkv);
  const int rest = (int)(blockIdx.x / (unsigned)hkv);
  const int tile = a.tiles - 1 - rest % a.tiles;  // longest causal rows first
  const int b = rest / a.tiles;

  const int q0 = a.cu_q_lens[b];
  const int n = a.cu_q_lens[b + 1] - q0;  // new queries of the sequence
  const int L = a.seq_lens[b];
  const int ctx = L - n;
  const int p0 = tile * NP;               // first local position of the workgroup
  if (p0 >= n || L <= 0) return;
  const int pend = min(p0 + NP, n);
  const int Hq = hkv * G;

  // ---- this lane's row and its visible key range ---------------------------------
  const int row = lane % kRows;                  // column of the MFMA results
  const int grp = lane / kRows;                  // 0/1: half of the 64 lanes
  const int wg_row = wave * kRows + row;
  const int p_loc = p0 + wg_row / G;             // local query position
  const int hh = wg_row % G;
  const bool row_ok = p_loc < n;
  const int qpos = ctx + min(p_loc, n - 1);      // absolute position
  const int hi = a.causal ? qpos : L - 1;        // last visible key
  const int lo = a.window > 0 ? max(0, qpos - a.window + 1) : 0;
  // keys the workgroup needs
  const int wg_hi = a.causal ? ctx + pend - 1 : L - 1;
  const int wg_lo = a.window > 0 ? max(0, ctx + p0 - a.window + 1) : 0;
  int t_first = wg_lo / kTile;
  int t_last = wg_hi / kTile;
  // this row's partial result in a split launch (computed where used: kept live through
  // the main loop it cost registers)
  auto ws_row = [&]() {
    return ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * kWgRows + wg_row;
  };
  if (a.nsplit > 1) {
    const int T = (L + kTile - 1) / kTile;
    t_first = max(t_first, (int)((int64_t)blockIdx.y * T / a.nsplit));
    t_last = min(t_last, (int)((int64_t)(blockIdx.y + 1) * T / a.nsplit) - 1);
    if (t_first > t_last) {  // none of the workgroup's keys in this split (uniform)
      if (grp == 0)
        *reinterpret_cast<float2*>(a.ws_ml + 2 * ws_row()) = make_float2(-INFINITY, 0.0f);
      return;
    }
  }
  const int npages = (L + kPage - 1) / kPage;
  const int* bt = a.block_table + (int64_t)b * a.bt_stride;
  // per-wave bounds for the mask decision
  const int w_hi_min = __builtin_amdgcn_readfirstlane(
      a.causal ? ctx + min(p0 + (wave * kRows) / G, n - 1) : L - 1);
  const int w_lo_max = __builtin_amdgcn_readfirstlane(
      a.window > 0 ? max(0, ctx + min(p0 + (wave * kRows + kRows - 1) / G, n - 1) -
                                a.window + 1)
                   : 0);

  // tiles every row of the wave sees whole: no key below w_lo_max, none above w_hi_min,
  // none past the sequence end
  const int t_clean_lo = (w_lo_max + kTile - 1) / kTile;
  const int t_clean_hi = min(w_hi_min + 1, L) / kTile - 1;

  // ---- direct loads -----------------------------------------------------------------
  auto issue_ids = [&](int c) {  // page ids of id chunk c, one per thread
    const int idx = min((t_first + kIdTiles * c) * kTilePages + tid, npages - 1);
    lds_load4(bt + idx, lds_offset(&ids_lds[c & 1][64 * wave]));
  };
  // Wave w issues load instructions w, w + 4, ... of the tile's K and V: instruction
  // q covers page q / PI, 64-chunk block jj = q % PI of it (jj is the same for all of
  // a wave's instructions).  Per-lane offsets inside the page:
  const int jj = wave % LY::PI;
  const int wpg = LY::PI == kWaves ? 0 : wave / LY::PI;  // first page of the wave
  // per-lane byte offsets inside a page (block jj included)
  uint32_t k_voff;
  {
    const int o = 64 * jj + lane;  // chunk inside the K page
    const int t = o / LY::NC, r = o % LY::NC;
    const int c = 2 * ((r / 2) ^ LY::phi(t)) + r % 2;
    k_voff = (uint32_t)((t - 64 * jj / LY::NC) * D + 16 * c + 1024 * jj);
  }
  const uint32_t v_voff = 16u * lane + 1024u * jj;
  // the four page ids of tile t (past the last tile: those of the last tile, whose
  // re-load is harmless), in one LDS read
  auto tile_ids_raw = [&](int t) {
    const int rel = min(t, t_last) - t_first;
    return *reinterpret_cast<const int4*>(
        &ids_lds[(rel / kIdTiles) & 1][(rel % kIdTiles) * kTilePages]);
  };
  auto uniform_ids = [](const int4 v) {
    return make_int4(__builtin_amdgcn_readfirstlane(v.x), __builtin_amdgcn_readfirstlane(v.y),
                     __builtin_amdgcn_readfirstlane(v.z), __builtin_amdgcn_readfirstlane(v.w));
  };
  auto tile_ids = [&](int t) { return uniform_ids(tile_ids_raw(t)); };
  // This wave's load instruction k of a tile covers block jj of page (kWaves / PI) k +
  // wpg.  The byte offsets of those pages (the same in the K and V pools: their pages
  // have one size, 16 D bytes) are computed once per tile, as independent scalar
  // chains (a dependent chain per load would cost its latency on every load).
  struct PageOffs {
    uint64_t o[LY::W];
  };
  auto page_offsets = [&](const int4 id4) {
    PageOffs p;
#pragma unroll
    for (int k = 0; k < LY::W; ++k) {
      const int pg = (kWaves / LY::PI) * k + wpg;
      const int id = pg == 0 ? id4.x : pg == 1 ? id4.y : pg == 2 ? id4.z : id4.w;
      p.o[k] = (uint64_t)(uint32_t)(id * hkv + g) * (uint64_t)(16 * D);
    }
    return p;
  };
  // K side: k < W covers K block k, then (per-token-head) the scales of the tile with
  // (uniform) page ids id4; V side: V block k.
  auto issue_k = [&](int k, uint8_t* slot, const PageOffs& po, const int4 id4) {
    if (k < LY::W) {
      const int pg = (kWaves / LY::PI) * k + wpg;
      lds_load16s(a.k_pages + po.o[k], k_voff,
                  lds_offset(slot + 16 * (pg * LY::KPC + 64 * jj)));
    } else if constexpr (kPTH) {  // waves 0/2: K scales, 1/3: V scales (2, 3 repeat)
      const int page = lane / kPage;
      const int id = page == 0 ? id4.x : page == 1 ? id4.y : page == 2 ? id4.z : id4.w;
      const int64_t idx = ((int64_t)id * hkv + g) * kPage + lane % kPage;
      const bool kside = wave % 2 == 0;
      lds_load4((kside ? a.k_scales : a.v_scales) + idx,
                lds_offset(slot + (kside ? LY::KS_OFF : LY::VS_OFF)));
    }
  };
  auto issue_v = [&](int k, uint8_t* slot, const PageOffs& po) {
    const int pg = (kWaves / LY::PI) * k + wpg;
    lds_load16s(a.v_pages + po.o[k], v_voff, lds_offset(slot + 16 * (pg * D + 64 * jj)));
  };
  // This wave's direct loads done, then every wave's (a compiler barrier on each side
  // keeps the LDS reads of the new contents after it).
  auto publish = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // Slots past the sequence end were never written (any bytes, NaN included): zero
  // the V bytes of a tile that ends past it before anyone reads them (its scales are
  // masked where they are read).
  const int t_partial = L % kTile ? L / kTile : -1;  // the tile the sequence ends in
  auto scrub_v = [&](int t, uint8_t* st) {
    if (t != t_partial) return;
    const int valid = L - t * kTile;  // keys of the tile below the sequence end
    for (int ch = tid; ch < LY::VT_CHUNKS; ch += kThreads) {
      const int keep = min(max(valid - (ch / D) * kPage, 0), kPage);  // tokens kept
      if (keep < kPage) {
        uint32_t* w = reinterpret_cast<uint32_t*>(st + 16 * ch);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int kq = min(max(keep - 4 * q, 0), 4);
          w[q] &= kq >= 4 ? 0xFFFFFFFFu : ((1u << (8 * kq)) - 1u);
        }
      }
    }
    barrier_lds();
  };
  // this KV head's layer scales: per-KV-head arrays or the per-tensor pair
  float k_scale_g = a.k_scale, v_scale_g = a.v_scale;
  if constexpr (!kPTH) {
    if (a.head_scales) {
      k_scale_g = a.k_scales[g];
      v_scale_g = a.v_scales[g];
    }
  }
  const float qk_base = a.q_scale * a.sm_log2 * (kPTH ? 1.0f : k_scale_g);
  // Every wave derives the per-key factors of a resident tile into its own block;
  // v_ref (the running V scale maximum) moves here, tile by tile, identically in
  // every wave.
  float vref_run = 0.0f;
  auto read_scales = [&](const uint8_t* kslot, float& ks, float& vs) {
    if constexpr (kPTH) {
      ks = reinterpret_cast<const float*>(kslot + LY::KS_OFF)[lane];
      vs = reinterpret_cast<const float*>(kslot + LY::VS_OFF)[lane];
    }
  };
  auto derive = [&](int t, uint8_t* fb, float ks, float vs) {
    if constexpr (kPTH) {
      // keys past the sequence end hold unwritten scales: take them as 0
      if (t * kTile + lane >= L) ks = vs = 0.0f;
      // V scales are >= 0: compare bits
      vref_run = __uint_as_float(
          max(__float_as_uint(vref_run), wave_max_u32(__float_as_uint(vs))));
      // P' factor and its reciprocal (hardware reciprocals: any f works as long as
      // the row sum maps P' back with the same f, up to rounding)
      const float f = vref_run > 0.0f ? vs * __builtin_amdgcn_rcpf(vref_run * a.prob_scale)
                                      : 0.0f;
      reinterpret_cast<float*>(fb + LY::CF_OFF)[lane] = ks * qk_base;
      reinterpret_cast<float*>(fb + LY::FV_OFF)[lane] = f;
      reinterpret_cast<float*>(fb + LY::IF_OFF)[lane] = f > 0.0f ? __builtin_amdgcn_rcpf(f) : 0.0f;
    }
  };

  // ---- query codes: B operand of S^T = K . Q^T -----------------------------------
  // lane holds row `row`, dims 64 ks + 32 grp + 0..31 as 32 e4m3 codes per step.
  v8i qb[KS];
  {
    const uint16_t* qrow = a.q + ((int64_t)(q0 + min(p_loc, n - 1)) * Hq + g * G + hh) * D;
    auto quantise = [&](auto enc) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4* src = reinterpret_cast<const uint4*>(qrow + 64 * ks + 32 * grp);
        uint32_t w[8];
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
          const uint4 x = src[c4];
          const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            uint32_t word = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t bits = (xs[2 * h + e / 2] >> (16 * (e % 2))) & 0xFFFFu;
              word |= enc(bf16_bits_to_float(bits)) << (8 * e);
            }
            w[2 * c4 + h] = row_ok ? word : 0u;
          }
        }
        qb[ks] = (v8i){(int)w[0], (int)w[1], (int)w[2], (int)w[3],
                       (int)w[4], (int)w[5], (int)w[6], (int)w[7]};
      }
    };
    // x / 1.0 == x exactly, so a unit scale skips the division
    if (a.q_scale == 1.0f) quantise([](float f) { return e4m3_encode(f); });
    else quantise([&](float f) { return e4m3_quantize(f, a.q_scale); });
  }

  // ---- running state ---------------------------------------------------------------
  v16f o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = (v16f){};
  float m = -INFINITY;   // reference row maximum (log2 units), same in both lane halves
  // this lane's part of the row sum: p units (per-token-head mode) or P' units
  // (per-tensor mode, where P' = p / prob_scale for every key)
  float lam = 0.0f;
  float vref = kPTH ? 0.0f : v_scale_g;  // v_ref the accumulator is expressed in
  // per-lane operand bases inside a stage
  // K operand: MFMA row `row` of key block kb is key tile_key(32 kb + row): page
  // 2 kb + (row / 4) % 2, token 4 (row / 8) + row % 4; dim step ks reads chunks
  // 4 ks + 2 grp and the next (one 32-byte pair).  Key block 1 is two pages on.
  int k_addr[KS];
  {
    const int tr = 4 * (row / 8) + row % 4;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      k_addr[ks] = 16 * (((row / 4) % 2) * LY::KPC + LY::NC * tr +
                                     2 * ((2 * ks + grp) ^ LY::phi(tr)));
  }
  constexpr int K_KB = 16 * 2 * LY::KPC;
  // V^T operand: channel 32 db + row; bytes 0-15 = page grp, 16-31 = page 2 + grp
  const int v_lane = 16 * (grp * D + row);
  constexpr int V_HI = 16 * 2 * D;
  const int s_lane = 4 * 16 * grp;  // factors of lane group grp inside a block
  const float pmul = 1.0f / a.prob_scale;

  // S^T = K . Q^T of a resident tile, for the two 32-key blocks
  auto qk = [&](const uint8_t* buf, v16f (&sc)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sc[kb] = (v16f){};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int off = k_addr[ks] + K_KB * kb;
        const uint4 x0 = lds_read<uint4>(buf, off);
        const uint4 x1 = lds_read<uint4>(buf, off + 16);
        const v8i ka = {(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                        (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        sc[kb] = mfma(ka, qb[ks], sc[kb]);
      }
    }
  };

  // Scores of a tile in log2 units relative to the current reference maximum,
  // x = s * CF - msafe, for the 4 keys of group w (key block w / 4, registers
  // 4 (w % 4) .. + 3).  Lane group grp, register r of key block kb holds key
  // 32 kb + 16 grp + r.
  auto scale_group = [&](int w, const uint8_t* buf, const v16f (&sc)[2], float msafe,
                         float (&x)[32]) {
    const int kb = w / 4, q4 = w % 4;
    float4 c4;
    if constexpr (kPTH)
      c4 = lds_read<float4>(buf, LY::CF_OFF + s_lane + 16 * (8 * kb + q4));
    else
      c4 = make_float4(qk_base, qk_base, qk_base, qk_base);
    const float cc[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) x[4 * w + e] = fmaf(sc[kb][4 * q4 + e], cc[e], -msafe);
  };
  // Masks the keys of tile t a row must not see (-inf); returns the lane's maximum.
  auto mask_max = [&](int t, float (&x)[32]) {
    const int kbase = t * kTile;
    if (t < t_clean_lo || t > t_clean_hi) {
      // visible keys relative to this lane's first key: element (kb, r) is key
      // 32 kb + r of that range.  The empty asm keeps the per-key tests inside this
      // (rarely taken) branch instead of hoisted into every tile.
      int lo_r = lo - (kbase + 16 * grp);
      int hi_r = hi - (kbase + 16 * grp);
      if (!row_ok || hi_r < lo_r) lo_r = hi_r = 1 << 20;  // nothing visible
      asm volatile("" : "+v"(lo_r), "+v"(hi_r));
      const uint32_t span = (uint32_t)(hi_r - lo_r);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const bool vis = (uint32_t)(32 * kb + r - lo_r) <= span;
          x[16 * kb + r] = vis ? x[16 * kb + r] : -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 32; ++i) mx = fmaxf(mx, x[i]);
    return mx;
  };

  // prologue: page ids of the first chunk; K of tiles t_first, t_first + 1 and V of
  // t_first resident; then K of t_first + 2 and V of t_first + 1 in flight (the order
  // the loop's waits count on); factors of t_first derived (iteration t derives those
  // of tile t + 1).
  issue_ids(0);
  wait_vmcnt<0>();
  barrier_lds();
  {
    const int4 i0 = tile_ids(t_first), i1 = tile_ids(t_first + 1);
    const PageOffs o0 = page_offsets(i0), o1 = page_offsets(i1);
#pragma unroll
    for (int k = 0; k < PER_K; ++k) issue_k(k, k_lds[0], o0, i0);
#pragma unroll
    for (int k = 0; k < PER_K; ++k) issue_k(k, k_lds[1], o1, i1);
#pragma unroll
    for (int k = 0; k < PER_V; ++k) issue_v(k, v_lds[0], o0);
    wait_vmcnt<0>();
    publish();
    scrub_v(t_first, v_lds[0]);
    const int4 i2 = tile_ids(t_first + 2);
    const PageOffs o2 = page_offsets(i2);
#pragma unroll
    for (int k = 0; k < PER_K; ++k) issue_k(k, k_lds[2], o2, i2);
#pragma unroll
    for (int k = 0; k < PER_V; ++k) issue_v(k, v_lds[1], o1);
  }
  {
    float ks = 0.0f, vs = 0.0f;
    read_scales(k_lds[0], ks, vs);
    derive(t_first, f_lds[wave][0], ks, vs);
  }

  // The tile loop, specialised on how P' is formed from p: PM 0: p * factor; PM 1:
  // the same clamped to the e4m3 maximum; PM 2: p itself (per-tensor mode with
  // prob_scale 1).  Iteration t: the scores of tile t + 1 are computed on the matrix
  // cores while the vector unit forms P' of tile t; then the P.V product of tile t
  // runs while the row sum and the next tile's scaled scores are formed.
  auto main_loop = [&](auto pm_tag) {
    constexpr int PM = decltype(pm_tag)::value;
    // ---- operand queue: chunk c < NQK is S^T MFMA c (K operand of tile t + 1, P'
    // factors of tile t), chunk NQK + db is P.V MFMA db (V operand of tile t, row-sum
    // factors of tile t, score factors of tile t + 1).  Operands are read QD chunks
    // ahead, across the barrier and into the next iteration.
    constexpr int NQK = 2 * KS;          // MFMAs of S^T per tile
    constexpr int WQ = 8 / NQK;          // P' words per phase-1 chunk
    constexpr int WV = 8 / DB;           // row-sum words / score groups per phase-2 chunk
    constexpr int NCH = NQK + DB;
    // queue depth (chunks read ahead): two.  With MFMAs free to move across chunk
    // boundaries (below) the scheduler hoists the reads itself; a depth of four measured
    // the same (within 1%, builds timed round-robin) and costs registers
    constexpr int QD = 2;
    // head_dim 256 has the registers to carry the queue over the loop's back edge, so
    // the next tile's first operand reads are issued at the end of this one (others
    // issue them at the top of the iteration)
    constexpr bool kCrossQueue = D == 256;
    static_assert(QD <= NQK && QD <= DB, "queue depth");
    // across the back edge chunk c of the next tile is read from the slot it was loaded
    // into, (c + NCH - QD) % QD, as c % QD: equal only when QD divides NCH
    static_assert(NCH % QD == 0, "queue depth must divide the chunk count");
    // the loads in phase-1 chunks 1 .. NQK - 1 (chunk 0 would wait for the page-id
    // read), LPC per chunk: K of tile t + 3, then V of tile t + 2
    constexpr int NLD = PER_K + PER_V;
    constexpr int LPC = NQK > 1 ? (NLD + NQK - 2) / (NQK - 1) : NLD;
    // The chunk that waits for K of tile t + 2 / V of tile t + 1 and publishes them: the
    // start of phase 2, or -- head_dim 256 per-token-head, where the loads' latency shows
    // -- the last chunk before the back-edge queue first reads K of tile t + 2 (1468 ->
    // 1441 us; per-tensor 1206 -> 1239 us the other way, so it keeps the early one).
    constexpr int kPublishChunk = kCrossQueue && kPTH ? NCH - QD - 1 : NQK;
    static_assert(kPublishChunk >= NQK && kPublishChunk + QD <= NCH + (kCrossQueue ? 0 : QD),
                  "publish before the first read of K of tile t + 2");
    struct Chunk {
      v8i op;
      float4 f2[WV];  // score factors (phase-2 chunks, queued mode)
    };
    auto k_operand = [&](const uint8_t* kb, int i) {  // key block i % 2, dim step i / 2
      const int off = k_addr[i / 2] + K_KB * (i % 2);
      const uint4 x0 = lds_read<uint4>(kb, off);
      const uint4 x1 = lds_read<uint4>(kb, off + 16);
      return (v8i){(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                   (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
    };
    auto v_operand = [&](const uint8_t* vb, int db) {
      const int off = v_lane + 16 * 32 * db;
      const uint4 x0 = lds_read<uint4>(vb, off);
      const uint4 x1 = lds_read<uint4>(vb, off + V_HI);
      return (v8i){(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                   (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
    };
    // per-key factors of word / score group w (keys 32 (w / 4) + 16 grp + 4 (w % 4) ..)
    auto factor = [&](const uint8_t* fb, int region, int w, float uniform) {
      if constexpr (kPTH) return lds_read<float4>(fb, region + s_lane + 16 * (8 * (w / 4) + w % 4));
      else return make_float4(uniform, uniform, uniform, uniform);
    };
    // chunk c of an iteration whose K operand tile is in kb, V operand tile in vb,
    // factors of its tile in fb and of the next tile in fbn
    auto load_chunk = [&](int c, const uint8_t* kb, const uint8_t* vb, const uint8_t* fb,
                          const uint8_t* fbn, Chunk& q) {
      if (c < NQK) {
        q.op = k_operand(kb, c);
      } else {
        const int db = c - NQK;
        q.op = v_operand(vb, db);
        if constexpr (!kLateFactors) {
#pragma unroll
          for (int u = 0; u < WV; ++u) q.f2[u] = factor(fbn, LY::CF_OFF, WV * db + u, qk_base);
        }
      }
    };

    float x[32];
    uint32_t pw[8] = {0, 0, 0, 0, 0, 0, 0, 0};  // P' codes of the current tile
    {
      v16f sc[2];
      qk(k_lds[0], sc);
#pragma unroll
      for (int w = 0; w < 8; ++w) scale_group(w, f_lds[wave][0], sc, 0.0f, x);
    }
    Chunk cq[QD];
    if constexpr (kCrossQueue) {
#pragma unroll
      for (int c = 0; c < QD; ++c)
        load_chunk(c, k_lds[1], v_lds[0], f_lds[wave][0], f_lds[wave][1], cq[c]);
    }

    PageOffs offs_v = page_offsets(tile_ids(t_first + 2));  // page offsets of tile t + 2
    int4 ids_k_raw = tile_ids_raw(t_first + 3);  // of tile t + 3, read one tile ahead
    // One tile step.  R = (t - t_first) & 3, the tile's place in the four-slot rings.
    // The chained form passes it as a compile-time constant: the loop below is unrolled
    // by hand over the ring period (the compiler does not unroll a loop with a barrier
    // in it), so every slot address is a constant.  The explicit-flush form, whose
    // extra zeroed accumulators leave no registers for four copies, keeps the rolled
    // loop with R a plain integer.
    auto step = [&](auto r_tag, const int t) {
      const int R = static_cast<int>(r_tag);
      const int rel = t - t_first;
      const uint8_t* kb1 = k_lds[(R + 1) & 3];  // K of tile t + 1
      const uint8_t* kb2 = k_lds[(R + 2) & 3];  // K of tile t + 2 (published mid-way)
      uint8_t* const kb3 = k_lds[(R + 3) & 3];  // K of tile t + 3 goes here
      const uint8_t* vb0 = v_lds[R];            // V of tile t
      uint8_t* const vb1 = v_lds[(R + 1) & 3];  // V of tile t + 1 (published mid-way)
      uint8_t* const vb2 = v_lds[(R + 2) & 3];  // V of tile t + 2 goes here
      uint8_t* const fb0 = f_lds[wave][R & 1];        // factors of tile t
      uint8_t* const fb1 = f_lds[wave][(R + 1) & 1];  // factors of tile t + 1
      // V of tile t (published by the previous barrier) is first read in phase 1
      if (rel > 0) scrub_v(t, v_lds[R]);
      const float vr = vref_run;  // v_ref after tile t (before tile t + 1 is derived)
      // scales of tile t + 1 (resident since the previous barrier): read here, factors
      // written in chunk 1 (before the first read of them) or, with fewer than 4 S^T
      // chunks, right away
      float dks = 0.0f, dvs = 0.0f;
      read_scales(kb1, dks, dvs);
      if constexpr (kPTH && NQK < 4) derive(t + 1, fb1, dks, dvs);
      if constexpr (!kCrossQueue) {
#pragma unroll
        for (int c = 0; c < QD; ++c) load_chunk(c, kb1, vb0, fb0, fb1, cq[c]);
      }
      // P' factors and their reciprocals of tile t, lane i of row 2 grp + h holding key
      // 32 kb + 16 grp + i in register kb: score register r of key block kb takes its
      // factor from lane r of its row
      float fvb[2] = {pmul, pmul}, ifb[2] = {1.0f, 1.0f};
      if constexpr (kPTH) {
        const float* fv = reinterpret_cast<const float*>(fb0 + LY::FV_OFF) + 16 * grp + lane % 16;
        const float* fi = reinterpret_cast<const float*>(fb0 + LY::IF_OFF) + 16 * grp + lane % 16;
        fvb[0] = fv[0];
        fvb[1] = fv[32];
        ifb[0] = fi[0];
        ifb[1] = fi[32];
      }
      if (R == 0 && rel % kIdTiles == 0) issue_ids(rel / kIdTiles + 1);  // kIdTiles % 4 == 0
      const int4 ids_k = uniform_ids(ids_k_raw);
      const PageOffs offs_k = page_offsets(ids_k);
      // masks and row maxima of tile t's scores
      float mx = mask_max(t, x);

      // ---- rescale when v_ref grew or a score passed the reference by the slack ----
      float fo = 1.0f;  // factor for o
      if constexpr (kPTH) {
        if (vr > vref) {
          fo = vref > 0.0f ? vref / vr : 0.0f;
          vref = vr;
        }
      }
      const bool first = m == -INFINITY;
      if (__builtin_amdgcn_ballot_w64(mx > (first ? -INFINITY : kSlack)) != 0) {
        // rows past the slack (or at their first visible keys) reset the reference
        // to their maximum minus kRefTop; rows of the same wave whose maximum is above
        // kRefTop move up with them (free: the wave rescales anyway)
        const float rmax = max_xor<kRows>(mx);  // whole row, relative
        const float delta = first ? (rmax == -INFINITY ? 0.0f : rmax - kRefTop)
                                  : fmaxf(0.0f, rmax - kRefTop);
        if (!first) {
          const float alpha = __builtin_amdgcn_exp2f(-delta);
          fo *= alpha;
          lam *= alpha;
        }
        m = first ? rmax - kRefTop : m + delta;
#pragma unroll
        for (int i = 0; i < 32; ++i) x[i] -= delta;
      }
      if (__builtin_amdgcn_ballot_w64(fo != 1.0f) != 0) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          if constexpr (!kValuAdd) asm volatile("" : "+a"(o[db]));
          o[db] *= fo;
          if constexpr (!kValuAdd) asm volatile("" : "+a"(o[db]));
        }
      }

      // ---- phase 1 (chunks 0 .. NQK - 1): S^T of tile t + 1 on the matrix cores; P' of
      // tile t (e4m3, in the B-operand layout) on the vector unit.  Barrier.  Phase 2
      // (chunks NQK ..): O^T += V^T . P'^T on the matrix cores; the row sum of the
      // rounded P' and the scaled scores of tile t + 1 (past the last tile: unused) on
      // the vector unit.  Each chunk holds one MFMA and a share of the vector work;
      // scheduling barriers keep the matrix work and the loads in chunk order, so the
      // matrix cores, the vector unit and the LDS overlap.
      v16f sn[2] = {(v16f){}, (v16f){}};
      v8i pb;
      const float msafe = m == -INFINITY ? 0.0f : m;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const Chunk cur = cq[c % QD];
        if (c + QD < NCH)
          load_chunk(c + QD, kb1, vb0, fb0, fb1, cq[c % QD]);
        else if constexpr (kCrossQueue)  // the next tile's: K of t + 2, factors of t + 1
          load_chunk(c + QD - NCH, kb2, vb1, fb1, fb0, cq[c % QD]);
        if (c == NCH - 1) ids_k_raw = tile_ids_raw(t + 4);
        if (c >= 1 && c < NQK) {
#pragma unroll
          for (int u = 0; u < LPC; ++u) {
            const int k = (c - 1) * LPC + u;
            if (k < PER_K) issue_k(k, kb3, offs_k, ids_k);
            else if (k < NLD) issue_v(k - PER_K, vb2, offs_v);
          }
        }
        if constexpr (kPTH && NQK >= 4)
          if (c == 1) derive(t + 1, fb1, dks, dvs);
        if (c == kPublishChunk) {
          // K of tile t + 2 and V of tile t + 1 resident: wait for them (the loads of
          // K of tile t + 3 and V of tile t + 2 may stay in flight), publish
          wait_vmcnt<NLD>();
          publish();
        }
        if (c < NQK) {
          sn[c % 2] = mfma(cur.op, qb[c / 2], sn[c % 2]);
#pragma unroll
          for (int u = 0; u < WQ; ++u) {
            const int w = WQ * c + u;
            float pe[4], pq[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) pe[e] = __builtin_amdgcn_exp2f(x[4 * w + e]);
            if constexpr (PM == 2) {
#pragma unroll
              for (int e = 0; e < 4; ++e) pq[e] = pe[e];
            } else {
              if constexpr (kPTH) {
                mul4_row_bcast(pq, fvb[w / 4], 4 * (w % 4), pe);
              } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) pq[e] = pe[e] * pmul;
              }
              if constexpr (PM == 1) {
#pragma unroll
                for (int e = 0; e < 4; ++e) pq[e] = fminf(pq[e], kE4m3Max);
              }
            }
            // the two conversions fill bytes 0-1 and 2-3; the old contents are dead
            const uint32_t lo2 = __builtin_amdgcn_cvt_pk_fp8_f32(pq[0], pq[1], pw[w], false);
            pw[w] = __builtin_amdgcn_cvt_pk_fp8_f32(pq[2], pq[3], lo2, true);
          }
          if (c == NQK - 1)
            pb = (v8i){(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3],
                       (int)pw[4], (int)pw[5], (int)pw[6], (int)pw[7]};
        } else {
          const int db = c - NQK;
          if constexpr (kValuAdd) {
            // level 2 as an explicit flush: this chunk's 64-key sum into a zeroed
            // accumulator, then float32 vector adds into the running output
            const v16f part = mfma(cur.op, pb, (v16f){});
#pragma unroll
            for (int r = 0; r < 16; ++r) o[db][r] += part[r];
          } else {
            // level 2 on the matrix core: the float32 C operand chains the chunks
            o[db] = mfma(cur.op, pb, o[db]);
            // keep the accumulator in AGPRs across iterations: the (rare) rescale then
            // copies it out and back, instead of every iteration copying it to VGPRs.
            // head_dim 256 leaves the choice to the register allocator, which has the
            // registers to spare (pinned or not measured the same)
            if constexpr (D != 256) asm volatile("" : "+a"(o[db]));
          }
#pragma unroll
          for (int u = 0; u < WV; ++u) {
            const int w = WV * db + u;
            const float4 fc = kLateFactors ? factor(fb1, LY::CF_OFF, w, qk_base) : cur.f2[u];
            if constexpr (kPTH) {
              const float2_t d01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)pw[w], false);
              const float2_t d23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)pw[w], true);
              fmac4_row_bcast(lam, ifb[w / 4], 4 * (w % 4), d01.x, d01.y, d23.x, d23.y);
            } else {
              const half2_t h01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(pw[w], 1.0f, false);
              const half2_t h23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(pw[w], 1.0f, true);
              const half2_t one = {(_Float16)1.0f, (_Float16)1.0f};
              lam = __builtin_amdgcn_fdot2(h01, one, lam, false);
              lam = __builtin_amdgcn_fdot2(h23, one, lam, false);
            }
            const float cc[4] = {fc.x, fc.y, fc.z, fc.w};
            const int kb = w / 4, q4 = w % 4;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[4 * w + e] = fmaf(sn[kb][4 * q4 + e], cc[e], -msafe);
          }
        }
        // chunk boundary: global loads stay in chunk order; MFMAs, vector (the
        // exponentials included), scalar and LDS instructions may cross it (8,192 new on
        // 32,768, builds timed round-robin on one box, against a full barrier at every
        // boundary: head_dim 256 per-tensor 1441 -> 1270 us, head_dim 64 3-4%, head_dim
        // 256 per-token-head unchanged at ~1520 us)
        __builtin_amdgcn_sched_barrier(0x0002 | 0x0004 | 0x0008 | 0x0080 | 0x0100 | 0x0200 |
                                       0x0400);
      }
      offs_v = offs_k;
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    if constexpr (kValuAdd) {
      for (int t = t_first; t <= t_last; ++t) step((t - t_first) & 3, t);
    } else {
      int t = t_first;
      for (; t + 3 <= t_last; t += 4) {
        step(I0{}, t);
        step(I1{}, t + 1);
        step(I2{}, t + 2);
        step(I3{}, t + 3);
      }
      // the last (up to three) tiles: t - t_first is a multiple of 4 here
      if (t <= t_last) step(I0{}, t);
      if (t + 1 <= t_last) step(I1{}, t + 1);
      if (t + 2 <= t_last) step(I2{}, t + 2);
    }
  };
  static_assert(kIdTiles % 4 == 0, "page-id chunks start at ring position 0");
  if (a.prob_scale < 256.0f / kE4m3Max) {
    // P' = p * v_scale_j / (v_ref * prob_scale) can pass 448 only when prob_scale <
    // 2^8 / 448 (p <= 2^8, v_scale_j <= v_ref)
    main_loop(std::integral_constant<int, 1>{});
  } else if (!kPTH && a.prob_scale == 1.0f) {
    main_loop(std::integral_constant<int, 2>{});
  } else {
    main_loop(std::integral_constant<int, 0>{});
  }
  // drain the loads still in flight (re-loads past the last tile) before exit
  wait_vmcnt<0>();

  // ---- normalise and store: lane holds row `row`, dims 32 db + 8 (r/4) + 4 grp + r%4
  // O = sum_j P'_j v_code_j with P'_j ~ p_j v_scale_j / (v_ref prob_scale) and lam ~
  // sum_j p_j: out = O * v_ref * prob_scale / lam; per-tensor: P'_j ~ p_j / prob_scale
  // and lam ~ sum_j P'_j, out = O * v_scale / lam
  const float lsum = sum_xor<kRows>(lam);
  if (a.nsplit > 1) {  // partial result: O and the row sum, both relative to 2^m
    const float f = vref * (kPTH ? a.prob_scale : 1.0f);
    const int64_t wr = ws_row();
    float* wo = a.ws_o + wr * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<float4*>(wo + 32 * db + 8 * r4 + 4 * grp) =
            make_float4(o[db][4 * r4] * f, o[db][4 * r4 + 1] * f, o[db][4 * r4 + 2] * f,
                        o[db][4 * r4 + 3] * f);
    if (grp == 0) *reinterpret_cast<float2*>(a.ws_ml + 2 * wr) = make_float2(m, lsum);
    return;
  }
  const float inv = lsum > 0.0f ? vref * (kPTH ? a.prob_scale : 1.0f) / lsum : 0.0f;
  if (row_ok) {
    const int64_t orow = ((int64_t)(q0 + p_loc) * Hq + g * G + hh) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = 32 * db + 8 * r4 + 4 * grp;
        const float x0 = o[db][4 * r4] * inv, x1 = o[db][4 * r4 + 1] * inv;
        const float x2 = o[db][4 * r4 + 2] * inv, x3 = o[db][4 * r4 + 3] * inv;
        if (a.out_f32) {
          *reinterpret_cast<float4*>(static_cast<float*>(a.out) + orow + d0) =
              make_float4(x0, x1, x2, x3);
        } else {
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + orow + d0) =
              make_uint2(pack_bf16x2(x0, x1), pack_bf16x2(x2, x3));
        }
      }
  }
}

// Launches prefill_kernel<D, G, kPTH, kValuAdd> for a runtime group size (1, 2, 4, 8,
// 16), scale mode and accumulation form; one translation unit per head_dim
// (prefill_d64.hip, prefill_d128.hip, prefill_d256.hip) so they compile in parallel.
template <int D>
void launch_prefill_fp8(int G, bool per_token_head, bool valu_add, const PrefillArgs& args,
                        dim3 grid, hipStream_t st);

#define KVQ_DEFINE_PREFILL_LAUNCH(D)                                                   \
  template <>                                                                          \
  void launch_prefill_fp8<D>(int G, bool pth, bool valu, const PrefillArgs& args,      \
                             dim3 blocks, hipStream_t st) {                            \
    auto go = [&](auto g_tag) {                                                        \
      constexpr int GG = decltype(g_tag)::value;                                       \
      if (pth && valu) prefill_kernel<D, GG, true, true><<<blocks, kThreads, 0, st>>>(args);   \
      else if (pth) prefill_kernel<D, GG, true, false><<<blocks, kThreads, 0, st>>>(args);     \
      else if (valu) prefill_kernel<D, GG, false, true><<<blocks, kThreads, 0, st>>>(args);    \
      else prefill_kernel<D, GG, false, false><<<blocks, kThreads, 0, st>>>(args);             \
    };                                                                                 \
    switch (G) {                                                                       \
      case 1: go(std::integral_constant<int, 1>{}); break;                             \
      case 2: go(std::integral_constant<int, 2>{}); break;                             \
      case 4: go(std::integral_constant<int, 4>{}); break;                             \
      case 8: go(std::integral_constant<int, 8>{}); break;                             \
      case 16: go(std::integral_constant<int, 16>{}); break;                           \
    }                                                                                  \
  }

}  // namespace pf

}  // namespace kvq
