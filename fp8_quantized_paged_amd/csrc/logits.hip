// Paged query-key logits for a sparse-attention indexer: every cache token a query
// row may see, scored against each of the row's query heads, from an FP8 (e4m3) or
// bf16 paged cache ("vLLM Qwen3.8-Flash-Next: QSA Indexer ... FP8 support", section on
// the reference test of the decode/prefill selection: the top-k selection reads
// these scores, and with FP8 the scores are compared value by value, exact float32
// accumulation expected).
//
// Arithmetic.  FP8 cache: the query is quantised to e4m3 with q_scale (as in
// attention); codes are widened to f16 (exact: every e4m3 value is an f16 value) and
// S^T = K . Q^T runs on v_mfma_f32_32x32x16_f16: exact products, float32 sums; the
// result is scaled by q_scale * k_scale_j.  bf16 cache: q and k as bf16 on
// v_mfma_f32_32x32x16_bf16 (exact products, float32 sums), unscaled.
//
// Work split.  A workgroup owns one (request, KV head), one set of the request's 32-pair
// chunks (all of them unless the requests average more than 32 pairs) and `iters`
// consecutive 128-key tiles (1 to 12, chosen so that the launch has about two
// workgroups per CU), each of its 4 waves 32 keys of a tile (one 32-key MFMA block);
// the request's query rows times the group's query heads ("pairs") are the other MFMA
// operand, 32 at a time, staged once per chunk in LDS.  The tiles are software-pipelined: a wave loads
// all its page ids at once, then keeps two tiles' key rows in flight (a three-buffer
// register ring) while one is computed, so the block-table -> key -> store chain of
// dependent memory round trips is paid once per workgroup rather than once per tile.
// The contraction index is assigned so that lane group hg (lanes 32 hg ..) holds the
// contiguous half D/2 hg .. D/2 hg + D/2 - 1 of every key and
// query row: step s, element e <-> dim D/2 hg + 8 s + e (both operands agree, which
// is all a contraction needs), so each lane's operands are plain 16-byte loads.
// The loads of every tile are issued unconditionally and the output stores go through a
// buffer resource that drops the stores of lanes without output, so no branch hides a
// memory instruction from the compiler's wait counts: they then keep two tiles in
// flight (with the loads and stores behind branches each wait also drained the
// prefetched tiles; indexer shape, 8 cache copies rotated: 22.9 -> 21.8 us).
#include <algorithm>

#include "kvq_device.h"
#include "kvq_host.h"

namespace kvq {
namespace lg {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kTileKeys = kWaves * 32;  // keys per tile (32 per wave)
constexpr int kMaxIters = 12;           // tiles per workgroup, at most (2 page ids per lane pair)
// Workgroups a launch aims for: two per CU, all resident at once (two waves per SIMD),
// each keeping two tiles' keys in flight per wave (the kernel is bound per CU by the
// loads it has in flight, so the CU holding the most tiles sets the time).  Indexer
// shape (32 x 20,000 keys, D 128, 5,024 tiles), round-robin A/B: 512 workgroups of 10
// tiles, tile ring of three 22.2 us; one tile in flight: 736 workgroups of 7 tiles 26.2
// us, 640 of 8 28.5 us; the ring at three workgroups per CU 28.4 us.  Re-measured once
// the ring really kept two tiles in flight (see the header): 768 workgroups at three
// waves per SIMD 21.5 against 21.9 us, 1,024 23.2 us -- within the spread of the
// method for 768, so the target stays.
constexpr int kTargetGroups = 512;
// Requests with more than 32 (row, head) pairs on average (prefill-time selection:
// thousands of rows per request, 1 GB of scores and more) are also split over their
// 32-pair chunks, one per workgroup for the average request (a longer one loops), the
// tiles per workgroup then chosen for kTargetGroups over tiles x chunks.  A key tile is
// read once per chunk, from the L2 in practice (the workgroups sharing it run
// together).  Before, with the grid over tiles only, a request of 8,192 rows and
// 8,192 keys (4 query heads, 1 GB of scores) ran on 64 workgroups: 2.69 ms; split
// over chunks 448 us (at 4 and 16 chunks per workgroup 487 and 383 us, but a batch
// with one long request then waits on a few long workgroups: 404 and 684 us against
// 480 us at one).

struct LogitsArgs {
  const uint16_t* q;          // bf16 [rows][Hq][D]
  const int32_t* cu_rows;     // [B + 1]
  const int32_t* row_lens;    // [rows]
  const int32_t* seq_lens;    // [B]
  const int32_t* block_table;
  int32_t bt_stride;
  const uint8_t* k_pages;     // [P][Hkv][16][D] codes or bf16
  const float* k_scales;      // per-token-head [P][Hkv][16], per-KV-head [Hkv], or null
  int32_t num_kv_heads, num_q_heads;
  int32_t groups, iters;      // workgroups per (request, head, chunk set), tiles per workgroup
  int32_t cgroups;            // chunk sets per request: workgroup c takes chunks c, c + cgroups, ..
  float q_scale, k_scale;     // k_scale: per-tensor
  float* out;                 // [rows][Hq][out_stride]
  int32_t span_bytes;         // bytes a chunk's stores may reach from its first pair's row
  int32_t out_stride;
};

// 8 e4m3 codes (two words, byte order = element order) as 8 f16 values
__device__ __forceinline__ half8_t codes_to_f16(uint32_t lo, uint32_t hi) {
  const half2_t a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
  const half2_t b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
  const half2_t c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
  const half2_t d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
  return (half8_t){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// kMode: 0 per-tensor, 1 per-token-head, 2 per-KV-head (FP8 only)
// Two waves per SIMD: a launch's workgroups (two per CU) stay resident at once.  (A
// three-wave budget spilled the ring at head_dim 128.)
// kSt: 0 plain stores, 1 buffer stores, 2 buffer stores after a transpose in lane quads,
// 3 swapped operands with one dword store per pair row (group size a power of two)
template <int D, bool kFp8, int kMode, int kSt>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void
logits_kernel(const LogitsArgs a) {
  constexpr int ES = kFp8 ? 1 : 2;       // bytes per element
  constexpr int HB = D / 2 * ES;         // bytes of a lane group's half row
  constexpr int NV = HB / 16;            // 16-byte loads per half row
  constexpr int NS = D / 16;             // MFMA steps over D
  constexpr int QS = D * ES + 16;        // LDS stride of a pair's query row (padded)
  constexpr bool kBuf = kSt > 0;
  __shared__ __align__(16) uint8_t q_lds[32 * QS];
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
  const int lane = (int)threadIdx.x % kWave;
  const int col = lane % 32, hg = lane / 32;
  const int H = a.num_kv_heads;
  const int g = (int)(blockIdx.x % (unsigned)H);
  const int rest = (int)(blockIdx.x / (unsigned)H);
  const int grp0 = rest % a.groups;
  const int cset = (rest / a.groups) % a.cgroups;
  const int b = rest / a.groups / a.cgroups;
  const int G = a.num_q_heads / H;
  const int r0 = a.cu_rows[b];
  const int npairs = (a.cu_rows[b + 1] - r0) * G;
  if (npairs <= 32 * cset) return;       // whole workgroup: no barrier is skipped
  const int L = a.seq_lens[b];
  const int npages = (L + kPage - 1) / kPage;
  const int* bt = a.block_table + (int64_t)b * a.bt_stride;
  const int key_base = grp0 * a.iters * kTileKeys + wave * 32;  // wave's key of tile 0

  // All of the wave's page ids at once (lane j: page j % 2 of tile j / 2, j < 2 iters),
  // so no block-table round trip sits between one tile and the next.
  int pid_all = 0;
  {
    const int kw = key_base + (lane / 2) * kTileKeys;
    if (lane < 2 * a.iters && kw < a.out_stride && npages > 0)
      pid_all = bt[min(kw / kPage + (lane & 1), npages - 1)];
  }
  // per-tile loads of this wave: its lane's half row of key key_base + 128 it + col and
  // (per-token-head) the scale of key col of the wave's 32; the scales an output lane
  // needs (keys 8 q + 4 hg + e, register 4 q + e) come from those lanes at the store.
  // Tiles past the workgroup's range (it >= iters) are loaded but never computed.
  struct Tile {
    uint4 k[NV];
    float sc;
  };
  auto load_tile = [&](int it, Tile& t) {
    const int kw = key_base + it * kTileKeys;
    const bool tile_ok = it < a.iters && kw < a.out_stride;
    const int pi = 2 * min(it, kMaxIters - 1);
    const int pg[2] = {__builtin_amdgcn_readlane(pid_all, pi),
                       __builtin_amdgcn_readlane(pid_all, pi + 1)};
    const int key = kw + col;
    // Every lane issues its loads: a lane without a key (past the sequence or the
    // workgroup's range) reads the call's first query row instead (always there, 16-byte
    // aligned and at least D * ES bytes), and its garbage only reaches its own output
    // row, which is -inf or not stored.  A load behind a branch would make the compiler's
    // wait counts assume it may be missing, and each wait would then drain the
    // prefetched tiles as well.
    const bool ok = tile_ok && key < L;
    const int64_t slot = ((int64_t)(col < 16 ? pg[0] : pg[1]) * H + g) * kPage + key % kPage;
    if constexpr (kFp8 && kMode == 1)
      t.sc = *(ok ? a.k_scales + slot : reinterpret_cast<const float*>(a.q));
    else
      t.sc = 0.0f;
    const uint8_t* row =
        ok ? a.k_pages + slot * D * ES : reinterpret_cast<const uint8_t*>(a.q);
#pragma unroll
    for (int v = 0; v < NV; ++v) t.k[v] = *reinterpret_cast<const uint4*>(row + HB * hg + 16 * v);
  };
  // per-tensor / per-KV-head: one K scale for the head
  float k_scale_h = a.k_scale;
  if constexpr (kFp8 && kMode == 2) k_scale_h = a.k_scales[g];

  // 16-byte query pieces per thread and chunk (32 pairs x D / 8 pieces)
  constexpr int QI = (32 * (D / 8) + kThreads - 1) / kThreads;
  for (int p0 = 32 * cset; p0 < npairs; p0 += 32 * a.cgroups) {
    // The chunk's query rows are loaded first, then the first tiles' key rows, so the
    // key loads stay in flight while the query is encoded (memory operations complete
    // in order for the wait counter: a query load issued after them would wait for
    // them too).
    uint4 qw[QI];
#pragma unroll
    for (int u = 0; u < QI; ++u) {
      const int i = (int)threadIdx.x + kThreads * u;
      const int pp = i / (D / 8), c8 = i % (D / 8);  // pair, 8-element chunk
      const int p = p0 + pp;
      qw[u] = make_uint4(0, 0, 0, 0);
      if (i < 32 * (D / 8) && p < npairs)
        qw[u] = *reinterpret_cast<const uint4*>(
            a.q + ((int64_t)(r0 + p / G) * a.num_q_heads + g * G + p % G) * D + 8 * c8);
    }
    // Ring of kRing tile buffers, fully unrolled so every buffer stays a named register
    // set: kRing - 1 tiles' key rows are in flight while one is computed.
    constexpr int kRing = 3;
    Tile ring[kRing];
#pragma unroll
    for (int r = 0; r < kRing - 1; ++r) load_tile(r, ring[r]);
    // ---- the chunk's query rows into LDS (e4m3 codes for an FP8 cache, else bf16) ---
    __syncthreads();  // the previous chunk's operand reads are done
#pragma unroll
    for (int u = 0; u < QI; ++u) {
      const int i = (int)threadIdx.x + kThreads * u;
      if (i >= 32 * (D / 8)) break;
      const int pp = i / (D / 8), c8 = i % (D / 8);
      const uint4 w = qw[u];  // zero for columns without a pair
      if constexpr (kFp8) {
        // e4m3 codes of x / q_scale on the hardware converter (e4m3_quantize4: the same
        // codes as the integer encoder, NaN included; zero words give zero codes)
        const uint32_t xs[4] = {w.x, w.y, w.z, w.w};
        float f[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = bf16_bits_to_float((xs[e / 2] >> (16 * (e % 2))) & 0xFFFFu);
        *reinterpret_cast<uint2*>(q_lds + pp * QS + 8 * c8) =
            make_uint2(e4m3_quantize4(f, a.q_scale), e4m3_quantize4(f + 4, a.q_scale));
      } else {
        *reinterpret_cast<uint4*>(q_lds + pp * QS + 16 * c8) = w;
      }
    }
    const int p = p0 + col;
    const bool pair_ok = p < npairs;
    const int pr = r0 + (pair_ok ? p / G : 0), ph = g * G + (pair_ok ? p % G : 0);
    const int vis = pair_ok ? min(a.row_lens[pr], L) : 0;
    float* orow = a.out + ((int64_t)pr * a.num_q_heads + ph) * a.out_stride;
    // Stores (kSt 1, 2): a buffer resource from the chunk's first pair's output row,
    // a.span_bytes long (the host checked that every pair of a chunk stores inside it);
    // a lane with nothing to store takes an offset past that range, which the hardware
    // drops.  So the store needs no branch: every store is issued, and the compiler
    // counts it exactly in the waits for the key loads (a store behind a branch made it
    // wait for a prefetched tile too).  With kSt 0 (a chunk spanning 2 GB or more of
    // output) the stores are plain and conditional.
    const int64_t base_f = ((int64_t)(r0 + p0 / G) * a.num_q_heads + g * G + p0 % G) * a.out_stride;
    int rel_f = 0;  // this pair's row, in floats from base_f
    if constexpr (kSt == 1)
      rel_f = pair_ok ? (int)(((int64_t)pr * a.num_q_heads + ph) * a.out_stride - base_f) : 0;
    // kSt 2: stores go out after a 4 x 4 transpose within each quad of lanes (below):
    // store t of lane 4 m + j writes pair 4 m + t, so each lane needs the rows of the four
    // pairs of its quad (offsets in floats from base_f; -1 where the pair does not exist).
    int rel_q[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int pq = p0 + (col & ~3) + t;
      rel_q[t] = -1;
      if constexpr (kSt == 2)
        if (pq < npairs)
          rel_q[t] = (int)(((int64_t)(r0 + pq / G) * a.num_q_heads + g * G + pq % G) *
                               a.out_stride - base_f);
    }
    // kSt 3: the MFMA computes S = Q . K^T (query rows as the A operand), so register
    // 4 q4 + e of lane (col, hg) holds pair 8 q4 + 4 hg + e against key kw + col, and
    // a dword store of one register writes 128 contiguous bytes of each of two pair
    // rows.  With G a power of two (and p0 a multiple of 32), a pair's row offset from
    // base_f splits over the disjoint bit fields of 8 q4 + e and 4 hg:
    // rel(i) = ((i / G) Hq + i % G) out_stride is the per-lane rel(4 hg) plus a
    // per-register constant rel(8 q4 + e) (wave-uniform).  Pairs past the request's
    // last are dropped by the buffer's record count, which ends with the last valid
    // pair's row (rows grow with the pair index).
    const int lgG = __builtin_ctz((unsigned)G);
    auto rel_of = [&](int i) {
      return ((i >> lgG) * a.num_q_heads + (i & (G - 1))) * a.out_stride;
    };
    int vis_r[kSt == 3 ? 16 : 1];
    int minvis = 0, maxvis = 0;  // over the chunk's pairs (wave-uniform)
    int lane_rel = 0;            // rel(4 hg) + col
    uint32_t span = kBuf ? (uint32_t)a.span_bytes : 0u;
    if constexpr (kSt == 3) {
#pragma unroll
      for (int r = 0; r < 16; ++r) vis_r[r] = __shfl(vis, 8 * (r / 4) + 4 * hg + r % 4);
      int mn = pair_ok ? vis : 0x7FFFFFFF, mx = pair_ok ? vis : 0;
#pragma unroll
      for (int m = 1; m < 32; m <<= 1) {
        mn = min(mn, __shfl_xor(mn, m));
        mx = max(mx, __shfl_xor(mx, m));
      }
      minvis = __builtin_amdgcn_readfirstlane(mn);
      maxvis = __builtin_amdgcn_readfirstlane(mx);
      lane_rel = rel_of(4 * hg) + col;
      span = 4u * (uint32_t)(rel_of(min(32, npairs - p0) - 1) + a.out_stride);
    }
    const __amdgpu_buffer_rsrc_t orsrc =  // gfx9 word 3: 32-bit raw buffer
        __builtin_amdgcn_make_buffer_rsrc(a.out + base_f, 0, (int)span, 0x00020000);
    __syncthreads();
    // B operand of this lane (pair col): its half row, kept for all tiles
    const uint8_t* qrow = q_lds + col * QS + HB * hg;
    // converted once per chunk, not per tile
    half8_t qf[kFp8 ? NS : 1];
    bf16x8_t qbf[kFp8 ? 1 : NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if constexpr (kFp8) {
        const uint2 qc = *reinterpret_cast<const uint2*>(qrow + 8 * s);
        qf[s] = codes_to_f16(qc.x, qc.y);
      } else {
        qbf[s] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(qrow + 16 * s));
      }
    }
    // this wave's tiles: it < nt (a.iters, fewer where the row ends first)
    const int nt = min(a.iters, max(0, (a.out_stride - key_base + kTileKeys - 1) / kTileKeys));
    auto compute_store = [&](int it, const Tile& t) {
      const int kw = key_base + it * kTileKeys;
      v16f acc = (v16f){};
      if constexpr (kSt == 3) {
        // tiles no pair of the chunk sees skip the matrix work (acc 0, all -inf below);
        // tiles every pair sees in full skip the mask (both tests wave-uniform, and only
        // arithmetic sits under them: every store is issued)
        if (kw < maxvis) {
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            if constexpr (kFp8) {
              const uint4 kv = t.k[s / 2];
              const half8_t ka = (s & 1) ? codes_to_f16(kv.z, kv.w) : codes_to_f16(kv.x, kv.y);
              acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(qf[s], ka, acc, 0, 0, 0);
            } else {
              acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  qbf[s], __builtin_bit_cast(bf16x8_t, t.k[s]), acc, 0, 0, 0);
            }
          }
        }
        float sck = 1.0f;
        if constexpr (kFp8) sck = (kMode == 1 ? t.sc : k_scale_h) * a.q_scale;
        const int key = kw + col;
        float v[16];
        if (kw + 32 <= minvis) {
#pragma unroll
          for (int r = 0; r < 16; ++r) v[r] = acc[r] * sck;
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) v[r] = key < vis_r[r] ? acc[r] * sck : -INFINITY;
        }
        // keys at or past out_stride: an offset past the record count (no wrap: the
        // per-register part stays below 0x7FF00000)
        const uint32_t voff = key < a.out_stride ? 4u * (uint32_t)(lane_rel + kw) : 0x7FFFFFF0u;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t off = voff + 4u * (uint32_t)rel_of(8 * (r / 4) + r % 4);
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[r]), orsrc, (int)off, 0, 0);
        }
        return;
      }
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        if constexpr (kFp8) {
          const uint4 kv = t.k[s / 2];  // key bytes 8 s .. 8 s + 7 of the half row
          const half8_t ka = (s & 1) ? codes_to_f16(kv.z, kv.w) : codes_to_f16(kv.x, kv.y);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka, qf[s], acc, 0, 0, 0);
        } else {
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, t.k[s]),
                                                        qbf[s], acc, 0, 0, 0);
        }
      }
      // ---- scale, mask (keys past the row's visible length -> -inf), store -----------
      // (every lane takes part in the scale permutes; only pair lanes store)
      // logit of key kw + 8 q4 + 4 hg + e for pair col (register 4 q4 + e)
      auto scaled = [&](int q4, int e) {
        float sc = k_scale_h;
        if constexpr (kFp8 && kMode == 1) sc = __shfl(t.sc, 8 * q4 + 4 * hg + e);
        return kw + 8 * q4 + 4 * hg + e < vis ? acc[4 * q4 + e] * (kFp8 ? sc * a.q_scale : 1.0f)
                                              : -INFINITY;
      };
      if constexpr (kSt == 2) {
        float w[4][4];  // [key group q4][e]
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int k0 = kw + 8 * q4 + 4 * hg;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float sc = k_scale_h;
            if constexpr (kFp8 && kMode == 1) sc = __shfl(t.sc, 8 * q4 + 4 * hg + e);
            w[q4][e] = k0 + e < vis ? acc[4 * q4 + e] * (kFp8 ? sc * a.q_scale : 1.0f) : -INFINITY;
          }
        }
        // 4 x 4 transpose of the 16-byte groups within each lane quad (lane 4 m + j, slot
        // t <- lane 4 m + t, slot j), in two exchanges over bit 0 and bit 1 of the lane:
        // afterwards slot t holds keys kw + 8 j + 4 hg .. + 3 of pair 4 m + t, so store t
        // writes 128 contiguous bytes (keys kw .. kw + 31) of each of 8 pairs, not 32
        // bytes of each of 32.
        const bool b0 = lane & 1, b1 = lane & 2;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const float snd = b0 ? w[2 * k][e] : w[2 * k + 1][e];
            const float rcv = __int_as_float(
                __builtin_amdgcn_update_dpp(0, __float_as_int(snd), 0xB1, 0xF, 0xF, false));
            if (b0) w[2 * k][e] = rcv; else w[2 * k + 1][e] = rcv;
          }
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const float snd = b1 ? w[k][e] : w[k + 2][e];
            const float rcv = __int_as_float(
                __builtin_amdgcn_update_dpp(0, __float_as_int(snd), 0x4E, 0xF, 0xF, false));
            if (b1) w[k][e] = rcv; else w[k + 2][e] = rcv;
          }
        }
        const int kq = kw + 8 * (lane & 3) + 4 * hg;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
          const u32x4v bits = {__float_as_uint(w[t][0]), __float_as_uint(w[t][1]),
                               __float_as_uint(w[t][2]), __float_as_uint(w[t][3])};
          // 0x7FFFFFF0: past any span_bytes (< 0x7FF00000), without wrapping
          const int off = rel_q[t] >= 0 && kq < a.out_stride ? 4 * (rel_q[t] + kq) : 0x7FFFFFF0;
          __builtin_amdgcn_raw_buffer_store_b128(bits, orsrc, off, 0, 0);
        }
      } else {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int k0 = kw + 8 * q4 + 4 * hg;
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = scaled(q4, e);
          if constexpr (kSt == 1) {
            typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
            const u32x4v bits = {__float_as_uint(v[0]), __float_as_uint(v[1]),
                                 __float_as_uint(v[2]), __float_as_uint(v[3])};
            const int off = pair_ok && k0 < a.out_stride ? 4 * (rel_f + k0) : 0x7FFFFFF0;
            __builtin_amdgcn_raw_buffer_store_b128(bits, orsrc, off, 0, 0);
          } else if (pair_ok && k0 < a.out_stride) {  // out_stride % 4 == 0: all 4 or none
            *reinterpret_cast<float4*>(orow + k0) = make_float4(v[0], v[1], v[2], v[3]);
          }
        }
      }
    };
    int i0 = 0;
    for (; i0 + kRing <= nt; i0 += kRing) {
#pragma unroll
      for (int r = 0; r < kRing; ++r) {
        load_tile(i0 + r + kRing - 1, ring[(r + kRing - 1) % kRing]);
        compute_store(i0 + r, ring[r]);
        // keeps the next step's operand converts (and so the wait for its tile) from
        // being hoisted into this one
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int r = 0; r < kRing - 1; ++r)
      if (i0 + r < nt) compute_store(i0 + r, ring[r]);
  }
}

template <int D, bool kFp8, int kSt>
static void launch_mode_b(int mode, const LogitsArgs& args, unsigned blocks, hipStream_t st) {
  if (!kFp8)
    logits_kernel<D, false, 0, kSt><<<blocks, kThreads, 0, st>>>(args);
  else if (mode == KVQ_SCALE_PER_TOKEN_HEAD)
    logits_kernel<D, true, 1, kSt><<<blocks, kThreads, 0, st>>>(args);
  else if (mode == KVQ_SCALE_PER_KV_HEAD)
    logits_kernel<D, true, 2, kSt><<<blocks, kThreads, 0, st>>>(args);
  else
    logits_kernel<D, true, 0, kSt><<<blocks, kThreads, 0, st>>>(args);
}
template <int D, bool kFp8>
static void launch_mode(int mode, int store, const LogitsArgs& args, unsigned blocks,
                        hipStream_t st) {
  if (store == 3) launch_mode_b<D, kFp8, 3>(mode, args, blocks, st);
  else if (store == 2) launch_mode_b<D, kFp8, 2>(mode, args, blocks, st);
  else if (store == 1) launch_mode_b<D, kFp8, 1>(mode, args, blocks, st);
  else launch_mode_b<D, kFp8, 0>(mode, args, blocks, st);
}

template <int D>
static void launch_dtype(const kvq_cache_desc* c, int store, const LogitsArgs& args,
                         unsigned blocks, hipStream_t st) {
  if (c->dtype == KVQ_FP8_E4M3) launch_mode<D, true>(c->mode, store, args, blocks, st);
  else launch_mode<D, false>(c->mode, store, args, blocks, st);
}

}  // namespace lg
}  // namespace kvq

using namespace kvq;

extern "C" kvq_status kvq_paged_logits(const kvq_cache_desc* cache, const void* q,
                                       const int32_t* cu_rows, int32_t num_seqs,
                                       int32_t total_rows, int32_t num_q_heads, const int32_t* row_lens,
                                       const int32_t* block_table, int32_t block_table_stride,
                                       const int32_t* seq_lens, const kvq_scales* scales,
                                       float* out, int32_t out_stride, void* stream) {
  clear_error();
  if (kvq_status s = check_cache(cache)) return s;
  if (num_seqs < 0 || total_rows < 0 || num_q_heads <= 0 || out_stride < 0)
    return fail(KVQ_ERR_INVALID_ARG, "num_seqs %d total_rows %d num_q_heads %d out_stride %d",
                num_seqs, total_rows, num_q_heads, out_stride);
  if (num_q_heads % cache->num_kv_heads)
    return fail(KVQ_ERR_INVALID_ARG, "num_q_heads %d not a multiple of num_kv_heads %d",
                num_q_heads, cache->num_kv_heads);
  if (num_seqs == 0 || total_rows == 0 || out_stride == 0) return KVQ_OK;
  if (out_stride % 4)
    return fail(KVQ_ERR_INVALID_ARG, "out_stride %d is not a multiple of 4", out_stride);
  if (!q || !out || !cu_rows || !row_lens || !seq_lens || !block_table)
    return fail(KVQ_ERR_INVALID_ARG, "q, out, cu_rows, row_lens, seq_lens or block_table is NULL");
  if (((uintptr_t)q | (uintptr_t)out) & 15u)
    return fail(KVQ_ERR_INVALID_ARG, "q and out must be 16-byte aligned");
  if (block_table_stride <= 0) return fail(KVQ_ERR_INVALID_ARG, "block_table_stride <= 0");
  if (cache->dtype == KVQ_FP8_E4M3 && cache->mode == KVQ_SCALE_PER_TOKEN_HEAD &&
      ((uintptr_t)cache->k_scales & 15u))
    return fail(KVQ_ERR_INVALID_ARG, "k_scales must be 16-byte aligned");
  lg::LogitsArgs a;
  int64_t pairs = 0;  // (row, head) pairs of the average request, per key head
  a.q = static_cast<const uint16_t*>(q);
  a.cu_rows = cu_rows;
  a.row_lens = row_lens;
  a.seq_lens = seq_lens;
  a.block_table = block_table;
  a.bt_stride = block_table_stride;
  a.k_pages = static_cast<const uint8_t*>(cache->k_pages);
  a.k_scales = cache->k_scales;
  a.num_kv_heads = cache->num_kv_heads;
  a.num_q_heads = num_q_heads;
  {
    const int64_t tiles = (out_stride + lg::kTileKeys - 1) / lg::kTileKeys;
    // 32-pair chunks of the average request (the kernel reads the actual rows from
    // cu_rows; a request with more chunks than this loops over them)
    const int64_t G = num_q_heads / cache->num_kv_heads;
    pairs = (total_rows + num_seqs - 1) / num_seqs * G;
    const int64_t chunks = (pairs + 31) / 32;
    a.cgroups = (int)chunks;
    // tiles per workgroup for about kTargetGroups workgroups, then spread evenly
    const int64_t total = (int64_t)num_seqs * cache->num_kv_heads * tiles * a.cgroups;
    const int64_t iters = std::min<int64_t>(lg::kMaxIters, std::max<int64_t>(
        1, (total + lg::kTargetGroups - 1) / lg::kTargetGroups));
    a.groups = (int)((tiles + iters - 1) / iters);
    a.iters = (int)((tiles + a.groups - 1) / a.groups);
  }
  a.q_scale = 1.0f;
  a.k_scale = 1.0f;
  if (cache->dtype == KVQ_FP8_E4M3) {
    if (!scales) return fail(KVQ_ERR_INVALID_ARG, "scales is NULL");
    if (!(scales->q_scale > 0.0f))
      return fail(KVQ_ERR_INVALID_ARG, "q_scale must be > 0");
    if (cache->mode == KVQ_SCALE_PER_TENSOR && !(scales->k_scale > 0.0f))
      return fail(KVQ_ERR_INVALID_ARG, "k_scale must be > 0");
    a.q_scale = scales->q_scale;
    a.k_scale = cache->mode == KVQ_SCALE_PER_TENSOR ? scales->k_scale : 1.0f;
  }
  a.out = out;
  a.out_stride = out_stride;
  {
    // 32 consecutive (row, head) pairs of one key head lie within 31 / G + 2 output rows
    // of Hq * out_stride floats from the first; a span that a 32-bit buffer offset cannot
    // cover takes the plain-store kernel (span_bytes 0)
    const int64_t G = num_q_heads / cache->num_kv_heads;
    const int64_t span = (31 / G + 2) * (int64_t)num_q_heads * out_stride * 4;
    a.span_bytes = span < 0x7FF00000 ? (int32_t)span : 0;
  }
  // store form: plain where a chunk's rows span 2 GB or more; else buffer stores, for
  // chunks of more than 8 pairs written row-contiguously: a store of the plain layout
  // touches 32 rows at 32 bytes each (8,192 rows x 8,192 keys, 4 heads: 404 us), the
  // lane-quad transpose makes it 8 rows at 128 bytes (243 us) and the swapped operands
  // 2 rows at 128 bytes with a fifth of the VALU work per tile (same in short bursts;
  // in 60-launch bursts 213-215 against 240-243 us, which clock down under the
  // heavier form).  The swapped form needs a power-of-two group; with 8 pairs or
  // fewer (one row per request, group 4) the plain layout stays (17.6 us against
  // 19.4 us transposed: most of the tile's lanes have no pair).
  const int64_t Gq = num_q_heads / cache->num_kv_heads;
  const int store = a.span_bytes == 0 ? 0 : pairs <= 8 ? 1 : (Gq & (Gq - 1)) == 0 ? 3 : 2;
  const int64_t blocks = (int64_t)num_seqs * cache->num_kv_heads * a.groups * a.cgroups;
  if (blocks > 0x7FFFFFFF) return fail(KVQ_ERR_INVALID_ARG, "grid too large");
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (cache->head_dim) {
    case 64: lg::launch_dtype<64>(cache, store, a, (unsigned)blocks, st); break;
    case 128: lg::launch_dtype<128>(cache, store, a, (unsigned)blocks, st); break;
    case 256: lg::launch_dtype<256>(cache, store, a, (unsigned)blocks, st); break;
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "logits launch: %s", hipGetErrorString(e));
  return KVQ_OK;
}
