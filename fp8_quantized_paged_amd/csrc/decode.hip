// Split-K paged GQA decode attention over an FP8 (or bf16) cache, with the split
// merge fused into the same launch.
//
// Method: "vLLM FP8 KV-Cache and Attention Quantization Update" (agentlenshq.com):
// FP8 e4m3 storage halves the bytes each decode step reads (section "Performance
// benchmarking"), attention runs on the FP8 values, partial sums are kept in true
// float32 registers (section "Two-level accumulation"), sliding-window layers may
// keep a bf16 cache (section "Hybrid attention and layer skipping"); the query is
// quantised inside the attention op (section "Kernel and fusion optimizations").
//
// Work split.  A workgroup of four waves owns one (sequence b, KV head g, split s);
// a split is a run of at most 256 cache pages of the sequence's visible key range,
// dealt to the waves round-robin (wave w takes pages w, w+4, ...).  Each wave serves
// all G query heads of the group, so every cache byte is loaded and converted once.
//
// Per page (16 tokens) a wave does:
//   QK  - "token layout": D/16 lanes share one token row, each lane holding 16
//         channels (one 16-byte load of fp8 codes, two of bf16).  Codes become
//         exact bf16 values (hardware convert) and meet the query's bf16 values in
//         v_dot2_f32_bf16 (products exact, float32 sums).  The lane partials are
//         summed across the token's lanes by a DPP butterfly that leaves each
//         lane holding distinct (token, head) scores.
//   softmax - float32 online softmax in the log2 domain with a lazily moved
//         reference maximum: the wave rescales only when some score exceeds the
//         reference by more than 2^8, so the common page costs one ballot.
//   PV  - "channel layout": lane l owns channels l + 64*i and reads their 16-token
//         rows of the dim-major V tile (one 16-byte load per channel).
//         fp8 cache: codes become exact f16 values and the weights, rounded to
//         f16 (relative error <= 2^-11; the weights never exceed 2^8), enter
//         v_dot2_f32_f16 with float32 accumulation straight into the running
//         output.  Per-token V scales are folded into the weight's exponent
//         (w = 2^(score + log2 v_scale - m_v)) against a second lazily moved
//         reference m_v, so the f16 weights stay in range whatever the scales.
//         bf16 cache: float32 weights and float32 FMAs.
//   Weights travel from the score lanes to the channel lanes through LDS.
// Accumulation levels: within a page in the dot2/FMA chains, the split in float32
// registers, the four waves of a workgroup through LDS, and the splits of a
// (sequence, KV head) by the last workgroup to finish (float32, fixed order).
#include "kvq_device.h"
#include "kvq_host.h"

namespace kvq {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr int ilog2c(int x) { return x <= 1 ? 0 : 1 + ilog2c(x / 2); }
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.0f;  // log2 units: weights stay <= 256
constexpr int kWaves = 4;              // waves per workgroup
constexpr int kThreads = kWaves * kWave;
constexpr int kMaxPagesPerWave = 64;   // one block-table entry per lane
constexpr int kMaxPagesPerSplit = kWaves * kMaxPagesPerWave;
// Workgroups the automatic split size aims for: two per CU on 256 CUs, all of
// them resident at once.
constexpr int kTargetWorkgroups = 512;
constexpr int kMaxAutoSplits = 32;
// s_waitcnt immediate (gfx9 encoding) that waits for every vector memory operation
// and leaves the LDS/export counters free.
constexpr int kWaitVmcnt0 = 0x0F70;
// Cache pages are read once per call: load them non-temporally (they bypass the
// caches' normal retention instead of evicting the block table, scales and query).
constexpr bool kStreamLoads = true;
constexpr int kXcds = 8;  // MI355X: workgroups are dealt to 8 XCDs round robin

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float v4f_t __attribute__((ext_vector_type(4)));
typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));

// Which form a decode instantiation takes (measured on MI355X over head_dim 64 / 128 /
// 256 and group sizes 1 .. 16).  The matrix-core form (see decode_kernel) costs a
// quarter of the vector-ALU work per page but reads K with one token row per lane
// (each 16-lane group touches 16 rows), so it wins where the vector form is
// ALU-bound: groups of 16, and groups of 8 up to head_dim 128.  The bf16 skip path
// always takes the vector form.
template <int D, int G, bool kFp8>
constexpr bool decode_uses_mfma() { return kFp8 && (G == 16 || (G == 8 && D <= 128)); }

__device__ __forceinline__ u32x4_t stream_load(const u32x4_t* p) {
  if constexpr (kStreamLoads) return __builtin_nontemporal_load(p);
  else return *p;
}
// Eight e4m3 codes (two dwords, byte order) -> their exact f16 values.
__device__ __forceinline__ half8_t codes8_to_f16(uint32_t lo, uint32_t hi) {
  const half2_t a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
  const half2_t b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
  const half2_t c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
  const half2_t d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
  return half8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ uint32_t stream_load(const uint32_t* p) {
  if constexpr (kStreamLoads) return __builtin_nontemporal_load(p);
  else return *p;
}

template <int D, int G, bool kFp8>
struct DecodeShape {
  static constexpr int LPT = D / 16;                // lanes per token row
  static constexpr int TPL = kWave / LPT;           // token groups per wave
  static constexpr int NT = kPage / TPL;            // token slots per lane per page
  static constexpr int NV = NT * G;                 // partial dots per lane
  static constexpr int LOG_LPT = ilog2c(LPT);
  static constexpr int LOG_NV = ilog2c(NV);
  static constexpr int NB = LOG_NV < LOG_LPT ? LOG_NV : LOG_LPT;  // butterfly steps
  static constexpr int NVL = NV >> NB;              // scores held per lane
  static constexpr int NAR = LOG_LPT - NB;          // plain all-reduce steps
  static constexpr int DPL = D / kWave;             // PV channels per lane
  static constexpr int KW = kFp8 ? 4 : 8;           // K dwords per lane per token slot
  static constexpr int VW = kFp8 ? 4 : 8;           // V dwords per channel row
  static constexpr int EB = kFp8 ? 1 : 2;           // element bytes
  // PV weights of one page in LDS: f16 [G][16] (fp8) or float [G][16] (bf16)
  static constexpr int W_WORDS = kFp8 ? G * kPage / 2 : G * kPage;
};

struct DecodeArgs {
  const uint16_t* q;
  int32_t num_kv_heads, splits, pps;
  int32_t max_len;  // the call's max_seq_len: longer device lengths are clamped to it
  const int32_t* block_table;
  int32_t bt_stride;
  const int32_t* seq_lens;
  const uint8_t* k_pages;
  const uint8_t* v_pages;
  const float* k_scales;  // per-token-head pools [P][Hkv][16], or per-KV-head [Hkv]
  const float* v_scales;
  float q_scale, k_scale, v_scale, sm_log2;  // per-tensor K/V scales
  int32_t head_scales;   // k_scales / v_scales are per-KV-head arrays
  int32_t window;
  float* o_part;      // [B*Hkv][splits][G][D]
  float* ml_part;     // [B*Hkv][splits][G][2]: reference max (log2), weight sum
  int32_t* counters;  // [B*Hkv] finished splits; zero between calls
  void* out;
  int32_t out_f32;
  // decode step only: the new token of each sequence (bf16 [B][Hkv][D]), written to
  // the cache at position seq_lens[b] - 1 before it is read; null for plain decode
  const uint16_t* k_new;
  const uint16_t* v_new;
};

// 8-byte agent-scope (device-coherent) stores and loads of float pairs: the split
// partials pass between workgroups on different XCDs, whose L2s are not coherent;
// per-access coherence avoids whole-cache write-back / invalidate fences.
__device__ __forceinline__ void store_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent2(float* p, float x, float y) {
  const uint64_t v = (uint64_t)__builtin_bit_cast(uint32_t, x) |
                     ((uint64_t)__builtin_bit_cast(uint32_t, y) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 load_agent2(const float* p) {
  const uint64_t v = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__builtin_bit_cast(float, (uint32_t)v),
                     __builtin_bit_cast(float, (uint32_t)(v >> 32)));
}

__device__ __forceinline__ void store_out(void* out, int32_t out_f32, int64_t i, float v) {
  if (out_f32)
    static_cast<float*>(out)[i] = v;
  else
    static_cast<uint16_t*>(out)[i] = (uint16_t)float_to_bf16_bits(v);
}

__device__ __forceinline__ float exp2_or_zero(float x) {
  return x == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(x);
}

// Butterfly over lane bits [LOG_LPT-1 .. LOG_LPT-NB]: each step halves the values a
// lane keeps and adds its partner's other half.
template <int NV, int LOG_LPT, int NB, int STEP>
__device__ __forceinline__ void butterfly(float (&v)[NV], int c) {
  if constexpr (STEP < NB) {
    constexpr int bit = LOG_LPT - 1 - STEP;
    constexpr int cnt = NV >> STEP;
    constexpr int half = cnt / 2;
    const bool up = (c >> bit) & 1;
#pragma unroll
    for (int k = 0; k < half; ++k) {
      const float keep = up ? v[k + half] : v[k];
      const float send = up ? v[k] : v[k + half];
      v[k] = keep + dpp_partner<bit>(send);
    }
    butterfly<NV, LOG_LPT, NB, STEP + 1>(v, c);
  }
}

// Plain all-reduce over the remaining low lane bits (group sizes below 4).
template <int NVL, int STEP, int NAR>
__device__ __forceinline__ void allreduce_low_bits(float (&v)[NVL]) {
  if constexpr (STEP < NAR) {
    constexpr int bit = NAR - 1 - STEP;
#pragma unroll
    for (int k = 0; k < NVL; ++k) v[k] += dpp_partner<bit>(v[k]);
    allreduce_low_bits<NVL, STEP + 1, NAR>(v);
  }
}

// Waves per SIMD the register allocation aims for: three where that costs no spills
// (head_dim 64 with per-tensor scales; the matrix-core form for groups of 8, except
// head_dim 128 with per-token-head scales), otherwise the compiler's choice.
template <int D, int G, bool kFp8, bool kPTH>
constexpr int decode_waves_per_eu() {
  if (decode_uses_mfma<D, G, kFp8>()) return G == 8 && (D == 64 || !kPTH) ? 3 : 1;
  return kFp8 && !kPTH && D == 64 && G <= 8 ? 3 : 1;
}
// Page buffers per wave (pages in flight + the one being computed): registers in the
// vector form; LDS slots (or registers, see decode_kernel) in the matrix-core form.
template <int D, int G, bool kFp8>
constexpr int decode_ring() { return decode_uses_mfma<D, G, kFp8>() ? 2 : 3; }

template <int D, int G, bool kFp8, bool kPTH, int kRing>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(
    decode_waves_per_eu<D, G, kFp8, kPTH>()))) void decode_kernel(const DecodeArgs a) {
  using S = DecodeShape<D, G, kFp8>;
  constexpr bool kMfma = decode_uses_mfma<D, G, kFp8>();
  constexpr int QW = G * D / 2;                  // query as bf16 pairs
  constexpr int NE4 = G * D / 4;                 // float4 groups of a (b, g) output
  // One-pass wave merge: every wave's G x D result fits an LDS slot of its own (32 KB for
  // the four), so one barrier separates the writes from a combine that all four waves
  // share; larger outputs take a tree through two slots.
  constexpr bool kOnePass = kWaves * G * D * 4 <= 32768;
  // wave-merge slots (floats): the waves' partial outputs, later the split merge's
  // (M, L, O) per float4 group of two waves
  constexpr int SLOTS = (kOnePass ? kWaves : kWaves / 2) * G * D;
  constexpr int MERGE = SLOTS > 12 * NE4 ? SLOTS : 12 * NE4;
  __shared__ uint32_t q_lds_all[kWaves][QW];
  __shared__ uint32_t w_lds_all[kWaves][S::W_WORDS];
  __shared__ float ml_lds[kWaves][G][2];
  __shared__ float merge_lds[MERGE];
  __shared__ int last_lds;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  // Workgroup order.  Pairs (b, s) run split-major (all sequences of split 0, then
  // split 1, ...), so the workgroups in flight together read neighbouring pages of
  // the pools.  The Hkv workgroups of one pair -- every KV head of the same pages --
  // are numbered 8 apart, which places them on one XCD (workgroups are dealt to the
  // eight XCDs round robin) so they stream the pages' head tiles side by side;
  // without a multiple of 8 pairs the heads of a pair are simply consecutive.  Within a
  // split the sequence index is rotated by the split, so that one sequence's splits go
  // to every XCD: numbered b = p % B, all splits of sequence b landed on XCD b % 8 when B
  // is a multiple of 8, and a batch with one long sequence streamed it on one XCD
  // (8 sequences, 40,000 + 7 x 1,000 tokens: 100 -> 51 us; equal lengths unchanged).
  const int H = a.num_kv_heads;
  const int npairs = (int)(gridDim.x / (unsigned)H);
  const int nb = npairs / a.splits;
  int bs, g;
  if (npairs % kXcds == 0) {
    const int blk = (int)blockIdx.x;
    bs = kXcds * (blk / (kXcds * H)) + blk % kXcds;
    g = (blk / kXcds) % H;
  } else {
    bs = (int)blockIdx.x / H;
    g = (int)blockIdx.x % H;
  }
  const int s = bs / nb;
  const int b = (bs % nb + nb - s % nb) % nb;
  const int ug = b * H + g;
  const int* bt = a.block_table + (int64_t)b * a.bt_stride;
  const int64_t row0 = (int64_t)ug * G;  // first output row: b * Hq + g * G
  // Issued before the sequence length is known: the query words of the group and,
  // for full attention (the split's pages then do not depend on the length), the
  // split's block-table entries; entries past the sequence are never used.
  int bt_lane = 0;
  if (a.window == 0) {
    const int idx = s * a.pps + wave + kWaves * lane;
    if (idx < min(s * a.pps + a.pps, a.bt_stride)) bt_lane = bt[idx];
  }
  constexpr int QPW = (QW + kWave - 1) / kWave;  // query words per lane
  uint32_t qraw[QPW];
  {
    const uint32_t* qsrc = reinterpret_cast<const uint32_t*>(a.q + row0 * D);
#pragma unroll
    for (int u = 0; u < QPW; ++u) {
      const int e = lane + u * kWave;
      qraw[u] = e < QW ? qsrc[e] : 0u;
    }
  }
  // A device length above the call's max_seq_len breaks the precondition the grid and
  // the workspace were sized by: such a sequence is read only up to max_seq_len (no
  // access past its block-table row, at most a.splits splits, so its merge still
  // runs and its counter returns to zero) and its new token, if any, is not written.
  const int L_dev = a.seq_lens[b];
  const int L = min(L_dev, a.max_len);
  const int lo = a.window > 0 ? max(0, L - a.window) : 0;
  const int pfirst = lo / kPage;
  const int pend = (L + kPage - 1) / kPage;
  const int ns = L > 0 ? min((pend - pfirst + a.pps - 1) / a.pps, a.splits) : 0;  // splits of (b, g)
  if (s >= ns) {
    if (s == 0) {  // empty sequence: zero output rows
      for (int e = tid; e < G * D; e += kThreads) store_out(a.out, a.out_f32, row0 * D + e, 0.0f);
    }
    return;
  }

  const int tg = lane / S::LPT;   // token group (QK layout)
  const int c = lane % S::LPT;    // channel chunk: channels 16c .. 16c+15
  uint32_t qv[G][8];              // bf16 pairs of channels 16c .. 16c+15, per head;
                                  // filled once the query is in LDS

  // score multiplier (log2 domain); per-token K scales multiply in per page
  // this KV head's layer scales: per-KV-head arrays or the per-tensor pair
  float k_scale_g = a.k_scale, v_scale_g = a.v_scale;
  if constexpr (kFp8 && !kPTH) {
    if (a.head_scales) {
      k_scale_g = a.k_scales[g];
      v_scale_g = a.v_scales[g];
    }
  }
  const float qk_base = kFp8 ? a.q_scale * a.sm_log2 * (kPTH ? 1.0f : k_scale_g) : a.sm_log2;

  // indices of the scores this lane holds after the butterfly
  int idx0 = 0;
#pragma unroll
  for (int st = 0; st < S::NB; ++st)
    idx0 += ((c >> (S::LOG_LPT - 1 - st)) & 1) * (S::NV >> (st + 1));
  const bool owner = (c & ((1 << S::NAR) - 1)) == 0;  // one lane per held score
  int hh_of[S::NVL], t_of[S::NVL];
#pragma unroll
  for (int k = 0; k < S::NVL; ++k) {
    const int n = idx0 + k;
    hh_of[k] = n % G;
    t_of[k] = tg + (n / G) * S::TPL;
  }

  // Running state.  m_all: per-head reference maximum of the scores (wave-uniform);
  // mv_all: reference of the V-weighted exponents (per-token-head scales only).
  float m_all[G], mv_all[G];
  float m_mine[S::NVL], mv_mine[S::NVL], l_mine[S::NVL];
  float acc[G][S::DPL];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    m_all[hh] = -INFINITY;
    mv_all[hh] = -INFINITY;
#pragma unroll
    for (int dd = 0; dd < S::DPL; ++dd) acc[hh][dd] = 0.0f;
  }
#pragma unroll
  for (int k = 0; k < S::NVL; ++k) {
    m_mine[k] = -INFINITY;
    mv_mine[k] = -INFINITY;
    l_mine[k] = 0.0f;
  }

  // this wave's pages of the split: pb + wave + kWaves * i, i < nwp
  const int pb = pfirst + s * a.pps;
  const int pe = min(pb + a.pps, pend);
  const int nwp = pe - pb > wave ? (pe - pb - wave + kWaves - 1) / kWaves : 0;
  if (a.window > 0) bt_lane = lane < nwp ? bt[pb + wave + kWaves * lane] : 0;
  uint32_t* w_lds = w_lds_all[wave];

  // Decode step: the wave that owns the page of position L - 1 stores the new token's
  // K and V (quantised exactly as the cache write does).  That page is the wave's last;
  // the store is issued before the load of that page -- after the first page loads
  // when the last page is not among them, so its latency overlaps them.  One wave's
  // memory operations are performed in program order (the AMDGPU memory model needs
  // no instruction for wavefront-scope ordering), so wavefront-scope fences, which
  // only keep the compiler from moving loads above the stores, order the two.
  bool app_owner = false;
  int app_page = 0;
  if (a.k_new != nullptr && L_dev == L) {
    const int lp = (L - 1) / kPage;
    const int rel = lp - pb;
    app_owner = rel >= 0 && lp < pe && rel % kWaves == wave;
    if (app_owner) app_page = __builtin_amdgcn_readlane(bt_lane, rel / kWaves);
  }
  auto append = [&]() {
    const int64_t tile = (int64_t)app_page * a.num_kv_heads + g;
    const int64_t src = ((int64_t)b * a.num_kv_heads + g) * D;
    if (lane < D / 8)
      store_token_row<D, kFp8, kPTH>(a.k_new + src, a.v_new + src, lane, tile,
                                     (L - 1) % kPage, const_cast<uint8_t*>(a.k_pages),
                                     const_cast<uint8_t*>(a.v_pages),
                                     const_cast<float*>(a.k_scales),
                                     const_cast<float*>(a.v_scales), k_scale_g, v_scale_g);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  // whether the first page loads (kRing - 1 of them) include the wave's last page
  const bool app_early = app_owner && nwp - 1 < kRing - 1;
  const bool app_late = app_owner && !app_early;
  if (app_early) append();

  float lw[G];  // this wave's weight sum per head (relative to m_all)
  if constexpr (kMfma) {
    // ---- matrix-core path ---------------------------------------------------------
    // Both products take f16 operands: every e4m3 value is exact in f16, and the f16
    // MFMA returns its sum rounded to float32 as a float32 dot product would (probe:
    // within 0.6 ulp of the sum of |products|), whereas the fp8 MFMA's internal sum
    // is off by up to ~1e-4 of the sum of |products| -- too coarse for scores that
    // span tens of log2 units over outlier channels.
    // Per page, S^T[token][head] = K . Q^T is one 16x16 accumulator (tokens = rows,
    // query heads = columns, heads past G are zero columns).  Lane (n = l % 16,
    // qg = l / 16) supplies row n of K (a quarter of the token's channels) and column
    // n of Q^T (the same quarter), and receives the scores of head n at tokens
    // 4 qg .. 4 qg + 3.  Those four scores, turned into weights, are exactly the lane's
    // part of the A operand of O = P . V (rows = heads, k = tokens 4 qg + r), so the
    // weights never leave the lane.  V enters as B (k = tokens, columns = 16
    // channels of one block): lane (n, qg) reads tokens 4 qg .. 4 qg + 3 of channel
    // 16 blk + n, one dword of the dim-major tile per block.  The running output is
    // D / 16 accumulators; lane (n, qg) holds heads 4 qg + r of channel 16 blk + n.
    const int n = lane & 15;
    const int qg = lane >> 4;
    const bool hvalid = n < G;
    constexpr int KB = D / 4;      // K bytes a lane supplies per page
    constexpr int NKV = KB / 16;   // 16-byte loads of them
    constexpr int NBLK = D / 16;   // PV accumulator blocks
    // Page inputs reach the operand layout -- which puts 16 token rows in every
    // 16-lane group -- in one of two ways (measured per shape):
    //  * staged (default): direct-to-LDS loads read the K and V tiles in order (each
    //    lane 16 bytes, a wave 1 KB of contiguous tile per load) into a per-wave ring
    //    of LDS slots, and the operand reads come from LDS.  Slot: K tile [16][D] |
    //    V tile [D][16] | 256 B of scales (lanes 0-15: K, 16-31: V, then repeats).
    //    The loads are counted by hand (NL per page; wait_vmcnt before a slot is read).
    //  * registers (head_dim 64, per-tensor scales): K is read in order, four lanes to
    //    a token row, and the lanes trade the pieces into place with lane permutes;
    //    V is read as one dword (4 tokens of one channel) per lane and block.  With
    //    every page coming from HBM (8 x 20,000 tokens, 64/8 heads) this runs 34.0 us
    //    against 36.5 us staged; staged wins only while the cache sits in the 256 MB
    //    last-level cache.
    constexpr bool kStage = !(D == 64 && !kPTH);
    constexpr int SLOT = kStage ? 32 * D + (kPTH ? 256 : 0) : 16;
    constexpr int NL = 2 * (D / 64) + (kPTH ? 1 : 0);
    __shared__ __attribute__((aligned(16))) uint8_t stage_all[kWaves][kRing][SLOT];
    uint8_t* const stage = stage_all[wave][0];
    struct RegPage {
      u32x4_t k;
      uint32_t v[NBLK];
    };
    RegPage regs[kStage ? 1 : kRing];
    auto mload = [&](int i, int slot) {
      const int page = __builtin_amdgcn_readlane(bt_lane, i);
      const int64_t tile = (int64_t)page * a.num_kv_heads + g;
      const uint8_t* kb = a.k_pages + tile * kPage * D;
      const uint8_t* vb = a.v_pages + tile * kPage * D;
      if constexpr (kStage) {
        uint8_t* dst = stage + slot * SLOT;
#pragma unroll
        for (int j = 0; j < D / 64; ++j)
          lds_load16s(kb, 16 * lane + 1024 * j, lds_offset(dst + 1024 * j));
#pragma unroll
        for (int j = 0; j < D / 64; ++j)
          lds_load16s(vb, 16 * lane + 1024 * j, lds_offset(dst + 16 * D + 1024 * j));
        if constexpr (kPTH)
          lds_load4((lane < 16 ? a.k_scales : a.v_scales) + tile * kPage + (lane & 15),
                    lds_offset(dst + 32 * D));
      } else {
        RegPage& r = regs[slot];
        r.k = stream_load(reinterpret_cast<const u32x4_t*>(kb) + lane);
        // dword 4 d + qg of the tile's channel-d row holds tokens 4 qg .. 4 qg + 3
        const uint32_t* vsrc = reinterpret_cast<const uint32_t*>(vb) + 4 * n + qg;
#pragma unroll
        for (int blk = 0; blk < NBLK; ++blk) r.v[blk] = stream_load(vsrc + 64 * blk);
      }
    };
    // every wave with pages issues kRing - 1 page loads up front (indices clamped to
    // its last page, so the counts below hold for any page count)
    if (nwp > 0) {
#pragma unroll
      for (int r = 0; r < kRing - 1; ++r) mload(min(r, nwp - 1), r);
    }
    if (app_late) append();

    // query: fused e4m3 quantisation into this wave's LDS copy, then the B operand
    // (f16 values of the codes; zero columns past the group)
    half8_t qb[D / 32];
    {
      uint8_t* q8 = reinterpret_cast<uint8_t*>(q_lds_all[wave]);
      const bool unit_q = a.q_scale == 1.0f;
#pragma unroll
      for (int u = 0; u < QPW; ++u) {
        const int e = lane + u * kWave;
        const float x0 = bf16_bits_to_float(qraw[u] & 0xFFFFu);
        const float x1 = bf16_bits_to_float(qraw[u] >> 16);
        const uint32_t c0 = unit_q ? e4m3_encode(x0) : e4m3_quantize(x0, a.q_scale);
        const uint32_t c1 = unit_q ? e4m3_encode(x1) : e4m3_quantize(x1, a.q_scale);
        if (e < QW) reinterpret_cast<uint16_t*>(q8)[e] = (uint16_t)(c0 | (c1 << 8));
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const uint32_t* qrow =
          reinterpret_cast<const uint32_t*>(q8 + (hvalid ? n : 0) * D + qg * KB);
      const uint32_t m = hvalid ? 0xFFFFFFFFu : 0u;
#pragma unroll
      for (int st = 0; st < D / 32; ++st)
        qb[st] = codes8_to_f16(qrow[2 * st] & m, qrow[2 * st + 1] & m);
    }

    // running state of head n (lanes n, n + 16, n + 32, n + 48 agree on m_h, mv_h)
    float m_h = -INFINITY, mv_h = -INFINITY, l_part = 0.0f;
    v4f_t acc_o[NBLK];
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk) acc_o[blk] = v4f_t{0.0f, 0.0f, 0.0f, 0.0f};

    auto mcompute = [&](int i, int slot) {
      const int t0 = (pb + wave + kWaves * i) * kPage;  // first position of the page
      const uint8_t* src = stage + slot * SLOT;
      u32x4_t kq[NKV];  // K row n, bytes qg * KB .. of it
      uint32_t vq[NBLK];  // tokens 4 qg .. 4 qg + 3 of channel 16 blk + n
      if constexpr (kStage) {
#pragma unroll
        for (int j = 0; j < NKV; ++j)
          kq[j] = *reinterpret_cast<const u32x4_t*>(src + n * D + qg * KB + 16 * j);
#pragma unroll
        for (int blk = 0; blk < NBLK; ++blk)  // bank-conflict free
          vq[blk] = *reinterpret_cast<const uint32_t*>(src + 16 * D + (16 * blk + n) * 16 +
                                                       4 * qg);
      } else {  // lane (n, qg) takes its K piece from lane 4 n + qg
        const RegPage& r = regs[slot];
        const int from = (4 * n + qg) * 4;
        kq[0].x = __builtin_amdgcn_ds_bpermute(from, (int)r.k.x);
        kq[0].y = __builtin_amdgcn_ds_bpermute(from, (int)r.k.y);
        kq[0].z = __builtin_amdgcn_ds_bpermute(from, (int)r.k.z);
        kq[0].w = __builtin_amdgcn_ds_bpermute(from, (int)r.k.w);
#pragma unroll
        for (int blk = 0; blk < NBLK; ++blk) vq[blk] = r.v[blk];
      }
      float ksc[4], vsc[4];
      if constexpr (kPTH) {
        const float4 k4 = *reinterpret_cast<const float4*>(src + 32 * D + 16 * qg);
        const float4 v4 = *reinterpret_cast<const float4*>(src + 32 * D + 64 + 16 * qg);
        ksc[0] = k4.x; ksc[1] = k4.y; ksc[2] = k4.z; ksc[3] = k4.w;
        vsc[0] = v4.x; vsc[1] = v4.y; vsc[2] = v4.z; vsc[3] = v4.w;
      }
      // ---- QK on the matrix cores: f16 values of the codes (exact), float32 sums ----
      // Step st takes bytes 8 st .. 8 st + 7 of each lane's quarter row, in K and Q.
      v4f_t sacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int st = 0; st < D / 32; ++st) {
        const u32x4_t kw = kq[st / 2];
        const half8_t ka = (st & 1) ? codes8_to_f16(kw.z, kw.w) : codes8_to_f16(kw.x, kw.y);
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qb[st], sacc, 0, 0, 0);
      }
      // ---- scale, mask, lazy rescale ---------------------------------------------
      const bool full = t0 >= lo && t0 + kPage <= L;  // wave-uniform
      float x[4], sv[4];
      bool over = false;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int pos = t0 + 4 * qg + rr;
        const bool vis = full || (pos >= lo && pos < L);
        const float sc = sacc[rr] * (kPTH ? qk_base * ksc[rr] : qk_base);
        x[rr] = vis ? sc : -INFINITY;
        over |= x[rr] > m_h + kRescaleSlack;
        if constexpr (kPTH) {
          // masked slots may hold unwritten scales: never take their logarithm
          sv[rr] = vis ? x[rr] + log2f(vsc[rr]) : -INFINITY;
          over |= sv[rr] > mv_h + kRescaleSlack;
        }
      }
      if (__builtin_amdgcn_ballot_w64(over && hvalid) != 0) {
        float pm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
        pm = max_xor<32>(max_xor<16>(pm));
        const float mn = fmaxf(m_h, pm);
        const float alpha = mn == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_h - mn);
        m_h = mn;
        l_part *= alpha;
        float beta = alpha;
        if constexpr (kPTH) {
          float pv = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
          pv = max_xor<32>(max_xor<16>(pv));
          const float mvn = fmaxf(mv_h, pv);
          beta = mvn == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(mv_h - mvn);
          mv_h = mvn;
        }
        // accumulator row 4 qg + rr is head 4 qg + rr, whose factor lane 4 qg + rr holds
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const float br = __shfl(beta, 4 * qg + rr);
          // in place, one register at a time (a plain product lets the compiler build
          // a scaled copy of every accumulator beside the originals)
#pragma unroll
          for (int blk = 0; blk < NBLK; ++blk)
            asm volatile("v_mul_f32 %0, %0, %1" : "+v"(acc_o[blk][rr]) : "v"(br));
        }
      }
      // ---- weights: the A operand of PV, f16 (they never exceed 2^8) ---------------
      half4_t pa;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const float p = __builtin_amdgcn_exp2f(x[rr] - m_h);
        l_part += p;
        const float w = kPTH ? __builtin_amdgcn_exp2f(sv[rr] - mv_h) : p;
        pa[rr] = hvalid ? (_Float16)w : (_Float16)0.0f;
      }
      // Slots past the sequence end (last page only) were never written: their bytes
      // may be any code, NaN included, and a zero weight times NaN is NaN.
      uint32_t vmask = 0xFFFFFFFFu;
      const int valid = L - t0;  // wave-uniform
      if (valid < kPage) {
        const int keep = min(max(valid - 4 * qg, 0), 4);
        vmask = keep >= 4 ? 0xFFFFFFFFu : ((1u << (8 * keep)) - 1u);
      }
      // ---- PV on the matrix cores: f16 x f16 (codes exact in f16), float32 sums ----
#pragma unroll
      for (int blk = 0; blk < NBLK; ++blk) {
        const uint32_t vw = vq[blk] & vmask;
        const half2_t lo2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(vw, 1.0f, false);
        const half2_t hi2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(vw, 1.0f, true);
        const half4_t vb = {lo2[0], lo2[1], hi2[0], hi2[1]};
        acc_o[blk] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, vb, acc_o[blk], 0, 0, 0);
      }
    };

    // Page i lives in slot i % kRing.  A full step refills the slot computed last
    // (its LDS reads done: lgkmcnt 0) and computes the next page once all but the
    // newest kRing - 1 page loads have landed.
    int i0 = 0;
    for (; i0 + kRing <= nwp; i0 += kRing) {
#pragma unroll
      for (int r = 0; r < kRing; ++r) {
        if constexpr (kStage) __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        mload(min(i0 + r + kRing - 1, nwp - 1), (r + kRing - 1) % kRing);
        if constexpr (kStage) wait_vmcnt<(kRing - 1) * NL>();
        mcompute(i0 + r, r);
      }
    }
    // the last pages (fewer than kRing, already loaded): the loads issued after
    // page i0 + r number kRing - 2 - r pages
    static_assert(kRing == 2 || kRing == 3, "staging ring of 2 or 3 slots");
    if (i0 < nwp) {
      if constexpr (kStage) wait_vmcnt<(kRing - 2) * NL>();
      mcompute(i0, 0);
    }
    if constexpr (kRing == 3) {
      if (i0 + 1 < nwp) {
        if constexpr (kStage) wait_vmcnt<0>();
        mcompute(i0 + 1, 1);
      }
    }

    // ---- per-head state to wave-uniform values; output to the channel layout ------
    const float lt = sum_xor<32>(sum_xor<16>(l_part));
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      m_all[hh] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                __builtin_bit_cast(int, m_h), hh));
      mv_all[hh] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                 __builtin_bit_cast(int, mv_h), hh));
      lw[hh] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                             __builtin_bit_cast(int, lt), hh));
    }
    if constexpr (kOnePass) {
      // the wave's result, scaled per head, straight into its slot ([G][D] layout):
      // accumulator row 4 qg + rr is head 4 qg + rr, channel 16 blk + n
      float fh[G];
#pragma unroll
      for (int hh = 0; hh < G; ++hh)
        fh[hh] = !kPTH ? v_scale_g
                       : (m_all[hh] == -INFINITY ? 0.0f
                                                 : __builtin_amdgcn_exp2f(mv_all[hh] - m_all[hh]));
      float* slot = merge_lds + wave * G * D;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int hr = 4 * qg + rr;
        float f = 0.0f;
#pragma unroll
        for (int hh = 0; hh < G; ++hh) f = hr == hh ? fh[hh] : f;
        if (hr < G) {
#pragma unroll
          for (int blk = 0; blk < NBLK; ++blk) slot[hr * D + 16 * blk + n] = acc_o[blk][rr] * f;
        }
      }
    } else {
    // two waves at a time through merge_lds (room for two G x D blocks)
#pragma unroll
    for (int round = 0; round < 2; ++round) {
      const bool mine = (wave >> 1) == round;
      float* slot = merge_lds + (wave & 1) * G * D;
      if (mine) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int hh = 4 * qg + rr;
          if (hh < G) {
#pragma unroll
            for (int blk = 0; blk < NBLK; ++blk) slot[hh * D + 16 * blk + n] = acc_o[blk][rr];
          }
        }
      }
      __syncthreads();
      if (mine) {
#pragma unroll
        for (int hh = 0; hh < G; ++hh)
#pragma unroll
          for (int dd = 0; dd < S::DPL; ++dd) acc[hh][dd] = slot[hh * D + lane + kWave * dd];
      }
      __syncthreads();
    }
    }  // two-round conversion
  } else {
  // One page's inputs for this lane: K rows of its token slots, V rows of its
  // channels, and the per-token scales of the scores it will hold.
  struct PageRegs {
    uint32_t kr[S::NT][S::KW];
    uint32_t vr[S::DPL][S::VW];
    float ksc[S::NVL], vsc[S::NVL];
  };

  auto load_page = [&](int i, PageRegs& r) {
    const int page = __builtin_amdgcn_readlane(bt_lane, i);
    const int64_t tile = (int64_t)page * a.num_kv_heads + g;
#pragma unroll
    for (int ts = 0; ts < S::NT; ++ts) {
      const int t = tg + ts * S::TPL;
      const u32x4_t* src = reinterpret_cast<const u32x4_t*>(
          a.k_pages + ((tile * kPage + t) * D + c * 16) * S::EB);
#pragma unroll
      for (int j = 0; j < S::KW / 4; ++j) {
        const u32x4_t x = stream_load(src + j);
        r.kr[ts][4 * j] = x.x; r.kr[ts][4 * j + 1] = x.y;
        r.kr[ts][4 * j + 2] = x.z; r.kr[ts][4 * j + 3] = x.w;
      }
    }
#pragma unroll
    for (int dd = 0; dd < S::DPL; ++dd) {
      const u32x4_t* src = reinterpret_cast<const u32x4_t*>(
          a.v_pages + ((tile * D + lane + kWave * dd) * kPage) * S::EB);
#pragma unroll
      for (int j = 0; j < S::VW / 4; ++j) {
        const u32x4_t x = stream_load(src + j);
        r.vr[dd][4 * j] = x.x; r.vr[dd][4 * j + 1] = x.y;
        r.vr[dd][4 * j + 2] = x.z; r.vr[dd][4 * j + 3] = x.w;
      }
    }
#pragma unroll
    for (int k = 0; k < S::NVL; ++k) {
      if constexpr (kFp8 && kPTH) {
        r.ksc[k] = a.k_scales[tile * kPage + t_of[k]];
        r.vsc[k] = a.v_scales[tile * kPage + t_of[k]];
      } else {
        r.ksc[k] = 1.0f;
        r.vsc[k] = 1.0f;
      }
    }
  };

  auto compute_page = [&](int i, const PageRegs& r) {
    const int lpage = pb + wave + kWaves * i;  // logical page
    // ---- QK partial dots -----------------------------------------------------
    float part[S::NV];
#pragma unroll
    for (int ts = 0; ts < S::NT; ++ts) {
      bf16x2_t kp[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if constexpr (kFp8) {
          kp[j] = (j & 1) ? e4m3x2_to_bf16x2<true>(r.kr[ts][j / 2])
                          : e4m3x2_to_bf16x2<false>(r.kr[ts][j / 2]);
        } else {
          kp[j] = as_bf16x2(r.kr[ts][j]);
        }
      }
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float x = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) x = dot2_bf16(as_bf16x2(qv[hh][j]), kp[j], x);
        part[ts * G + hh] = x;
      }
    }
    butterfly<S::NV, S::LOG_LPT, S::NB, 0>(part, c);
    float sc[S::NVL], sv[S::NVL];
#pragma unroll
    for (int k = 0; k < S::NVL; ++k) sc[k] = part[k];
    allreduce_low_bits<S::NVL, 0, S::NAR>(sc);

    // ---- scale, mask, lazy rescale ---------------------------------------------
    bool over = false;
#pragma unroll
    for (int k = 0; k < S::NVL; ++k) {
      const int pos = lpage * kPage + t_of[k];
      const bool vis = pos >= lo && pos < L;
      sc[k] = vis ? sc[k] * (qk_base * r.ksc[k]) : -INFINITY;
      over |= sc[k] > m_mine[k] + kRescaleSlack;
      if constexpr (kFp8 && kPTH) {
        // masked slots may hold unwritten scales: never take their logarithm
        sv[k] = vis ? sc[k] + log2f(r.vsc[k]) : -INFINITY;
        over |= sv[k] > mv_mine[k] + kRescaleSlack;
      }
    }
    if (__builtin_amdgcn_ballot_w64(over) != 0) {
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float x = -INFINITY, y = -INFINITY;
#pragma unroll
        for (int k = 0; k < S::NVL; ++k) {
          x = hh_of[k] == hh ? fmaxf(x, sc[k]) : x;
          if constexpr (kFp8 && kPTH) y = hh_of[k] == hh ? fmaxf(y, sv[k]) : y;
        }
        const float mn = fmaxf(m_all[hh], wave_max(x));
        const float alpha = mn == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_all[hh] - mn);
        m_all[hh] = mn;
        float beta = alpha;
        if constexpr (kFp8 && kPTH) {
          const float mvn = fmaxf(mv_all[hh], wave_max(y));
          beta = mvn == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(mv_all[hh] - mvn);
          mv_all[hh] = mvn;
        }
#pragma unroll
        for (int dd = 0; dd < S::DPL; ++dd) acc[hh][dd] *= beta;
#pragma unroll
        for (int k = 0; k < S::NVL; ++k) {
          if (hh_of[k] == hh) {
            l_mine[k] *= alpha;
            m_mine[k] = mn;
            if constexpr (kFp8 && kPTH) mv_mine[k] = mv_all[hh];
          }
        }
      }
    }

    // ---- weights -> LDS --------------------------------------------------------
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int k = 0; k < S::NVL; ++k) {
      const float p = __builtin_amdgcn_exp2f(sc[k] - m_mine[k]);
      float w = p;
      if constexpr (kFp8 && kPTH) w = __builtin_amdgcn_exp2f(sv[k] - mv_mine[k]);
      if (owner) {
        l_mine[k] += p;
        if constexpr (kFp8)
          reinterpret_cast<_Float16*>(w_lds)[hh_of[k] * kPage + t_of[k]] = (_Float16)w;
        else
          reinterpret_cast<float*>(w_lds)[hh_of[k] * kPage + t_of[k]] = w;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- PV ----------------------------------------------------------------------
    // Slots past the sequence end (last page only) were never written: their bytes
    // may be any code, NaN included, and a zero weight times NaN is NaN.
    uint32_t vw[S::DPL][S::VW];
#pragma unroll
    for (int dd = 0; dd < S::DPL; ++dd)
#pragma unroll
      for (int j = 0; j < S::VW; ++j) vw[dd][j] = r.vr[dd][j];
    const int valid = L - lpage * kPage;  // wave-uniform
    if (valid < kPage) {
      constexpr int TPW = 4 / S::EB;  // tokens per V word
#pragma unroll
      for (int j = 0; j < S::VW; ++j) {
        const int keep = min(max(valid - TPW * j, 0), TPW);
        const uint32_t msk = keep >= TPW ? 0xFFFFFFFFu : ((1u << (8 * S::EB * keep)) - 1u);
#pragma unroll
        for (int dd = 0; dd < S::DPL; ++dd) vw[dd][j] &= msk;
      }
    }
    if constexpr (kFp8) {
      half2_t vh[S::DPL][kPage / 2];
#pragma unroll
      for (int dd = 0; dd < S::DPL; ++dd)
#pragma unroll
        for (int j = 0; j < kPage / 2; ++j)
          vh[dd][j] = (j & 1)
              ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(vw[dd][j / 2], 1.0f, true)
              : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(vw[dd][j / 2], 1.0f, false);
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        half2_t wv[kPage / 2];
        const uint4 w0 = *reinterpret_cast<const uint4*>(w_lds + hh * (kPage / 2));
        const uint4 w1 = *reinterpret_cast<const uint4*>(w_lds + hh * (kPage / 2) + 4);
        wv[0] = __builtin_bit_cast(half2_t, w0.x); wv[1] = __builtin_bit_cast(half2_t, w0.y);
        wv[2] = __builtin_bit_cast(half2_t, w0.z); wv[3] = __builtin_bit_cast(half2_t, w0.w);
        wv[4] = __builtin_bit_cast(half2_t, w1.x); wv[5] = __builtin_bit_cast(half2_t, w1.y);
        wv[6] = __builtin_bit_cast(half2_t, w1.z); wv[7] = __builtin_bit_cast(half2_t, w1.w);
#pragma unroll
        for (int dd = 0; dd < S::DPL; ++dd) {
          float x = acc[hh][dd];
#pragma unroll
          for (int j = 0; j < kPage / 2; ++j) x = __builtin_amdgcn_fdot2(wv[j], vh[dd][j], x, false);
          acc[hh][dd] = x;
        }
      }
    } else {
      float vf[S::DPL][kPage];
#pragma unroll
      for (int dd = 0; dd < S::DPL; ++dd)
#pragma unroll
        for (int j = 0; j < kPage / 2; ++j) {
          vf[dd][2 * j] = bf16_bits_to_float(vw[dd][j] & 0xFFFFu);
          vf[dd][2 * j + 1] = bf16_bits_to_float(vw[dd][j] >> 16);
        }
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float pw[kPage];
#pragma unroll
        for (int j = 0; j < kPage / 4; ++j) {
          const float4 x = *reinterpret_cast<const float4*>(w_lds + hh * kPage + 4 * j);
          pw[4 * j] = x.x; pw[4 * j + 1] = x.y; pw[4 * j + 2] = x.z; pw[4 * j + 3] = x.w;
        }
#pragma unroll
        for (int dd = 0; dd < S::DPL; ++dd) {
          float x = acc[hh][dd];
#pragma unroll
          for (int t = 0; t < kPage; ++t) x = fmaf(pw[t], vf[dd][t], x);
          acc[hh][dd] = x;
        }
      }
    }
  };

  // Ring of kRing page buffers, fully unrolled so every buffer is a named register
  // set: kRing - 1 pages are in flight while one is computed.  The first loads go
  // out before the query is quantised, under one branch and with the index clamped (a
  // wave with one page loads it twice): with a branch around each load, the second
  // load's wait for its block-table entry also waited for the first page (8 x 20,000
  // Llama-shaped step 59.8 -> 59.4 us, window-128 layer 7.9 -> 7.5 us).
  PageRegs ring[kRing];
  if (nwp > 0) {
#pragma unroll
    for (int r = 0; r < kRing - 1; ++r) load_page(min(r, nwp - 1), ring[r]);
  }
  if (app_late) append();

  // ---- query of the group: fused e4m3 quantisation (fp8) or plain bf16 ----------
  // Every wave quantises the whole group into its own LDS copy, so only a wave-level
  // barrier separates the writes from the reads (a workgroup barrier would also wait
  // for the page loads already in flight).
  {
    uint32_t* q_lds = q_lds_all[wave];
    const bool unit_q = a.q_scale == 1.0f;
#pragma unroll
    for (int u = 0; u < QPW; ++u) {
      const int e = lane + u * kWave;
      uint32_t val = qraw[u];
      if constexpr (kFp8) {
        // x / 1.0 == x exactly, so the division is skipped for a unit scale
        const float x0 = bf16_bits_to_float(val & 0xFFFFu);
        const float x1 = bf16_bits_to_float(val >> 16);
        const uint32_t c0 = unit_q ? e4m3_encode(x0) : e4m3_quantize(x0, a.q_scale);
        const uint32_t c1 = unit_q ? e4m3_encode(x1) : e4m3_quantize(x1, a.q_scale);
        val = __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<false>(c0 | (c1 << 8)));
      }
      if (e < QW) q_lds[e] = val;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const uint4 x0 = *reinterpret_cast<const uint4*>(q_lds + (hh * D + c * 16) / 2);
      const uint4 x1 = *reinterpret_cast<const uint4*>(q_lds + (hh * D + c * 16) / 2 + 4);
      qv[hh][0] = x0.x; qv[hh][1] = x0.y; qv[hh][2] = x0.z; qv[hh][3] = x0.w;
      qv[hh][4] = x1.x; qv[hh][5] = x1.y; qv[hh][6] = x1.z; qv[hh][7] = x1.w;
    }
  }

  // Full steps: every step issues one page load (the index is clamped to the
  // wave's last page, so the final steps re-read it instead of branching) and
  // computes one page, so the loop body has no data-dependent branch around its
  // loads and the wait counts stay exact.
  int i0 = 0;
  for (; i0 + kRing <= nwp; i0 += kRing) {
#pragma unroll
    for (int r = 0; r < kRing; ++r) {
      load_page(min(i0 + r + kRing - 1, nwp - 1), ring[(r + kRing - 1) % kRing]);
      compute_page(i0 + r, ring[r]);
    }
  }
  // Remainder: fewer than kRing pages, all already loaded into slots 0 .. kRing-2.
#pragma unroll
  for (int r = 0; r < kRing - 1; ++r)
    if (i0 + r < nwp) compute_page(i0 + r, ring[r]);


#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    float x = 0.0f;
#pragma unroll
    for (int k = 0; k < S::NVL; ++k) x += (owner && hh_of[k] == hh) ? l_mine[k] : 0.0f;
    lw[hh] = wave_sum(x);
  }
  }  // vector-ALU path

  // ---- this wave's result relative to m_all: o = acc * f, l ------------------------
  // (the one-pass matrix-core form has already written its scaled result to LDS)
  if constexpr (!(kOnePass && kMfma)) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float f = kFp8 && !kPTH ? v_scale_g : 1.0f;
      if constexpr (kFp8 && kPTH)
        f = m_all[hh] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mv_all[hh] - m_all[hh]);
#pragma unroll
      for (int dd = 0; dd < S::DPL; ++dd) acc[hh][dd] *= f;
    }
  }

  const int64_t prow = (int64_t)ug * a.splits;  // split partial rows of (b, g)
  if constexpr (kOnePass) {
    // ---- merge the four waves in one pass (level 3, fixed order) ------------------
    // Element e = 64 w + l + 256 k of the G x D output (head e / D, the same for every
    // lane of wave w since D >= 64) is the sum over waves v = 0..3 of slot_v[e] scaled
    // from v's reference to the common one; wave w combines and stores its elements.
    if constexpr (!kMfma) {
      float* slot = merge_lds + wave * G * D;
#pragma unroll
      for (int hh = 0; hh < G; ++hh)
#pragma unroll
        for (int dd = 0; dd < S::DPL; ++dd) slot[hh * D + lane + kWave * dd] = acc[hh][dd];
    }
    if (lane == 0) {
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        ml_lds[wave][hh][0] = m_all[hh];
        ml_lds[wave][hh][1] = lw[hh];
      }
    }
    __syncthreads();
    constexpr int EPW = (G * D + kThreads - 1) / kThreads;  // elements per lane
    static_assert(D >= kWave, "one head per wave and element group");
    float val[EPW];
    float Mh[EPW], Lh[EPW];
#pragma unroll
    for (int k = 0; k < EPW; ++k) {
      const int e0 = kWave * wave + kThreads * k;   // wave-uniform
      const int hh = e0 < G * D ? e0 / D : 0;
      float mx = -INFINITY;
#pragma unroll
      for (int v = 0; v < kWaves; ++v) mx = fmaxf(mx, ml_lds[v][hh][0]);
      float sum = 0.0f, ls = 0.0f;
#pragma unroll
      for (int v = 0; v < kWaves; ++v) {
        const float mv = ml_lds[v][hh][0];
        const float c = mv == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mv - mx);
        ls += ml_lds[v][hh][1] * c;
        if (e0 < G * D) sum += merge_lds[v * G * D + e0 + lane] * c;
      }
      val[k] = sum;
      Mh[k] = mx;
      Lh[k] = ls;
    }
    if (ns == 1) {  // the only split: normalise and store directly
#pragma unroll
      for (int k = 0; k < EPW; ++k) {
        const int e0 = kWave * wave + kThreads * k;
        if (e0 < G * D)
          store_out(a.out, a.out_f32, row0 * D + e0 + lane, Lh[k] > 0.0f ? val[k] / Lh[k] : 0.0f);
      }
      return;
    }
#pragma unroll
    for (int k = 0; k < EPW; ++k) {
      const int e0 = kWave * wave + kThreads * k;
      if (e0 < G * D) {
        store_agent(a.o_part + (prow + s) * G * D + e0 + lane, val[k]);
        // one (M, L) pair per head, by the lane holding the head's first channel
        if ((e0 + lane) % D == 0)
          store_agent2(a.ml_part + ((prow + s) * G + (e0 + lane) / D) * 2, Mh[k], Lh[k]);
      }
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (wave == 0) {
      int done = 0;
      if (lane == 0)
        done = __hip_atomic_fetch_add(&a.counters[ug], 1, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
      done = __builtin_amdgcn_readfirstlane(done);
      if (lane == 0) last_lds = done == ns - 1;
    }
    __syncthreads();
    if (!last_lds) return;
  } else {

  // ---- merge the four waves (level 3, fixed order) --------------------------------
  if (lane == 0) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      ml_lds[wave][hh][0] = m_all[hh];
      ml_lds[wave][hh][1] = lw[hh];
    }
  }
  __syncthreads();
  float M[G], Lsum[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, ml_lds[w][hh][0]);
    M[hh] = mx;
    float ls = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      ls += ml_lds[w][hh][1] * exp2_or_zero(ml_lds[w][hh][0] == -INFINITY
                                                ? -INFINITY : ml_lds[w][hh][0] - mx);
    Lsum[hh] = ls;
    const float f = m_all[hh] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_all[hh] - mx);
#pragma unroll
    for (int dd = 0; dd < S::DPL; ++dd) acc[hh][dd] *= f;
  }
  // tree: waves [h, 2h) hand their sums to waves [0, h)
#pragma unroll
  for (int half = kWaves / 2; half >= 1; half /= 2) {
    if (wave >= half && wave < 2 * half) {
      float* slot = merge_lds + (wave - half) * G * D;
#pragma unroll
      for (int hh = 0; hh < G; ++hh)
#pragma unroll
        for (int dd = 0; dd < S::DPL; ++dd) slot[hh * D + lane + kWave * dd] = acc[hh][dd];
    }
    __syncthreads();
    if (wave < half) {
      const float* slot = merge_lds + wave * G * D;
#pragma unroll
      for (int hh = 0; hh < G; ++hh)
#pragma unroll
        for (int dd = 0; dd < S::DPL; ++dd) acc[hh][dd] += slot[hh * D + lane + kWave * dd];
    }
    __syncthreads();
  }

  if (ns == 1) {  // the only split: normalise and store directly
    if (wave == 0) {
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float inv = Lsum[hh] > 0.0f ? 1.0f / Lsum[hh] : 0.0f;
#pragma unroll
        for (int dd = 0; dd < S::DPL; ++dd)
          store_out(a.out, a.out_f32, (row0 + hh) * D + lane + kWave * dd, acc[hh][dd] * inv);
      }
    }
    return;
  }

  // ---- split partial -> workspace; the last split of (b, g) merges them all ---------
  // Partials are stored with agent-scope atomics, i.e. written through to the device
  // coherence point; the wave waits until they are performed before it counts itself
  // done, and the last workgroup reads them back with agent-scope loads.
  if (wave == 0) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float* o = a.o_part + ((prow + s) * G + hh) * D;
#pragma unroll
      for (int dd = 0; dd < S::DPL; ++dd) store_agent(o + lane + kWave * dd, acc[hh][dd]);
      if (lane == 0) store_agent2(a.ml_part + ((prow + s) * G + hh) * 2, M[hh], Lsum[hh]);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    int done = 0;
    if (lane == 0)
      done = __hip_atomic_fetch_add(&a.counters[ug], 1, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
    done = __builtin_amdgcn_readfirstlane(done);
    if (lane == 0) last_lds = done == ns - 1;
  }
  __syncthreads();
  if (!last_lds) return;
  }  // wave merge and split partial

  // Level-3 merge over the ns splits, by the last workgroup; lane l takes the float4
  // groups l, l + 64, ... of the G x D outputs, and batches of MB splits have all their
  // loads in flight at once.  When every split fits in one batch, wave 0 folds them all
  // in split order and the other waves leave (one round trip, no LDS tree); otherwise
  // wave w takes splits w, w + 4, ... (in order) and the four waves' (M, L, O) combine
  // in a fixed tree through LDS.  Only splits that exist are loaded.
  constexpr int E4L = (NE4 + kWave - 1) / kWave;
  // splits per batch (its loads all in flight; the page loop's registers are free here)
  constexpr int MB_REGS = 16;
  constexpr int MB = MB_REGS / E4L > 1 ? MB_REGS / E4L : 1;
  const bool solo = ns <= MB;  // workgroup-uniform
  if (solo && wave != 0) return;
  const int jfirst = solo ? 0 : wave;
  const int jstep = solo ? 1 : kWaves;
  float Mx[E4L], Ls[E4L];
  float4 Os[E4L];
#pragma unroll
  for (int k = 0; k < E4L; ++k) {
    Mx[k] = -INFINITY;
    Ls[k] = 0.0f;
    Os[k] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  }
  auto combine = [](float& m0, float& l0, float4& o0, float m1, float l1, float4 o1) {
    if (m1 == -INFINITY) return;
    const float mn = fmaxf(m0, m1);
    const float fa = m0 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m0 - mn);
    const float fb = __builtin_amdgcn_exp2f(m1 - mn);
    o0.x = o0.x * fa + o1.x * fb;
    o0.y = o0.y * fa + o1.y * fb;
    o0.z = o0.z * fa + o1.z * fb;
    o0.w = o0.w * fa + o1.w * fb;
    l0 = l0 * fa + l1 * fb;
    m0 = mn;
  };
  for (int j0 = jfirst; j0 < ns; j0 += jstep * MB) {
    float4 ov[MB][E4L];
    float2 mlv[MB][E4L];
#pragma unroll
    for (int u = 0; u < MB; ++u) {
      const int j = j0 + jstep * u;
      if (j < ns) {
#pragma unroll
        for (int k = 0; k < E4L; ++k) {
          const int e4 = min(lane + kWave * k, NE4 - 1);
          const float* op = a.o_part + (prow + j) * G * D + 4 * e4;
          const float2 lo2 = load_agent2(op), hi2 = load_agent2(op + 2);
          ov[u][k] = make_float4(lo2.x, lo2.y, hi2.x, hi2.y);
          mlv[u][k] = load_agent2(a.ml_part + ((prow + j) * G + (4 * e4) / D) * 2);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < MB; ++u)
#pragma unroll
      for (int k = 0; k < E4L; ++k)
        if (j0 + jstep * u < ns) combine(Mx[k], Ls[k], Os[k], mlv[u][k].x, mlv[u][k].y, ov[u][k]);
  }
  // tree over the waves: waves [h, 2h) hand their (M, L, O) to waves [0, h)
  float* mslot = merge_lds;                        // [2][NE4] M, L pairs
  float4* oslot = reinterpret_cast<float4*>(merge_lds + 4 * NE4);  // [2][NE4]
  if (!solo) {
#pragma unroll
    for (int half = kWaves / 2; half >= 1; half /= 2) {
      if (wave >= half && wave < 2 * half) {
#pragma unroll
        for (int k = 0; k < E4L; ++k) {
          const int e4 = lane + kWave * k;
          if (e4 < NE4) {
            const int i = (wave - half) * NE4 + e4;
            mslot[2 * i] = Mx[k];
            mslot[2 * i + 1] = Ls[k];
            oslot[i] = Os[k];
          }
        }
      }
      __syncthreads();
      if (wave < half) {
#pragma unroll
        for (int k = 0; k < E4L; ++k) {
          const int e4 = lane + kWave * k;
          if (e4 < NE4) {
            const int i = wave * NE4 + e4;
            combine(Mx[k], Ls[k], Os[k], mslot[2 * i], mslot[2 * i + 1], oslot[i]);
          }
        }
      }
      __syncthreads();
    }
  }
  if (wave == 0) {
#pragma unroll
    for (int k = 0; k < E4L; ++k) {
      const int e4 = lane + kWave * k;
      if (e4 < NE4) {
        const float inv = Ls[k] > 0.0f ? 1.0f / Ls[k] : 0.0f;
        const int64_t e = row0 * D + 4 * e4;
        store_out(a.out, a.out_f32, e, Os[k].x * inv);
        store_out(a.out, a.out_f32, e + 1, Os[k].y * inv);
        store_out(a.out, a.out_f32, e + 2, Os[k].z * inv);
        store_out(a.out, a.out_f32, e + 3, Os[k].w * inv);
      }
    }
    if (lane == 0)
      __hip_atomic_store(&a.counters[ug], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---- host side ----------------------------------------------------------------------

static int max_visible_pages(int32_t max_seq_len, int32_t window) {
  const int all = (max_seq_len + kPage - 1) / kPage;
  if (window <= 0) return all;
  const int win = (window + kPage - 1) / kPage + 1;
  return all < win ? all : win;
}

// Pages per split: enough splits that the grid fills the GPU with resident
// workgroups (kTargetWorkgroups), each wave getting at least two pages, and at most
// kMaxAutoSplits splits per (sequence, KV head): the merge of a unit's splits ends
// every launch, and beyond 32 it costs more than the extra workgroups gain (one
// 131,072-token sequence, 8 KV heads: 32 splits 51.6 µs, 64 splits 53.7 µs).
static int auto_pages_per_split(int32_t num_seqs, int32_t num_kv_heads, int max_pages) {
  const int64_t units = (int64_t)num_seqs * num_kv_heads;
  if (units <= 0 || max_pages <= 0) return 2 * kWaves;
  // a unit of at most four pages per wave (a sliding window, a short sequence) is one
  // split: extra splits would add the merge's round trips to a latency-bound launch
  // (gpt-oss-shaped window-128 layer, 9 pages: 2 splits -> 1)
  if (max_pages <= 4 * kWaves) return max_pages;
  int64_t splits = (kTargetWorkgroups + units - 1) / units;
  if (splits > kMaxAutoSplits) splits = kMaxAutoSplits;
  if (splits < 1) splits = 1;
  int64_t pps = (max_pages + splits - 1) / splits;
  if (pps < 2 * kWaves) pps = 2 * kWaves;
  if (pps > kMaxPagesPerSplit) pps = kMaxPagesPerSplit;
  return (int)pps;
}

struct DecodePlan {
  int pps;
  int splits;
  size_t bytes;  // 0: one split everywhere, no workspace used
};

// Workspace layout, the same for every call so that calls of any shape can share one
// buffer: the completion counters of unit u = b * Hkv + g (int32) sit at a fixed
// offset 4 u inside a fixed prefix of KVQ_DECODE_COUNTER_BYTES, and the split
// partials follow it.  A call's partials therefore never overlap a counter, and the
// counters a call leaves at zero stay zero for the next call, whatever its shape.
constexpr size_t kCounterBytes = KVQ_DECODE_COUNTER_BYTES;
static_assert(kCounterBytes == sizeof(int32_t) * KVQ_DECODE_MAX_SPLIT_UNITS, "counter prefix");

static kvq_status plan_decode(const kvq_cache_desc* cache, int32_t num_seqs,
                              int32_t num_q_heads, int32_t max_seq_len, int32_t window,
                              int32_t pages_per_split, DecodePlan* plan) {
  if (kvq_status s = check_cache(cache)) return s;
  if (num_seqs < 0 || num_q_heads <= 0 || max_seq_len < 0 || window < 0)
    return fail(KVQ_ERR_INVALID_ARG, "num_seqs %d num_q_heads %d max_seq_len %d window %d",
                num_seqs, num_q_heads, max_seq_len, window);
  if (num_q_heads % cache->num_kv_heads)
    return fail(KVQ_ERR_INVALID_ARG, "num_q_heads %d not a multiple of num_kv_heads %d",
                num_q_heads, cache->num_kv_heads);
  if (!supported_group(num_q_heads / cache->num_kv_heads))
    return fail(KVQ_ERR_UNSUPPORTED, "group size %d (1, 2, 4, 8, 16 are built)",
                num_q_heads / cache->num_kv_heads);
  if (pages_per_split < 0 || pages_per_split > kMaxPagesPerSplit)
    return fail(KVQ_ERR_INVALID_ARG, "pages_per_split %d (0..%d)", pages_per_split,
                kMaxPagesPerSplit);
  const int mp = max_visible_pages(max_seq_len, window);
  plan->pps = pages_per_split ? pages_per_split
                              : auto_pages_per_split(num_seqs, cache->num_kv_heads, mp);
  // at least one split: an all-empty batch still needs its zero output rows
  plan->splits = mp > 0 ? (mp + plan->pps - 1) / plan->pps : 1;
  const int64_t units = (int64_t)num_seqs * cache->num_kv_heads;
  if (plan->splits > 1 && units > KVQ_DECODE_MAX_SPLIT_UNITS)
    return fail(KVQ_ERR_UNSUPPORTED,
                "num_seqs * num_kv_heads = %lld > %d with %d splits (the workspace's "
                "counter prefix holds %d units)",
                (long long)units, KVQ_DECODE_MAX_SPLIT_UNITS, plan->splits,
                KVQ_DECODE_MAX_SPLIT_UNITS);
  plan->bytes = plan->splits > 1
                    ? kCounterBytes + (size_t)num_seqs * num_q_heads * plan->splits *
                                          (cache->head_dim + 2) * sizeof(float)
                    : 0;
  return KVQ_OK;
}

template <int D, int G, bool kFp8, bool kPTH>
static void launch(const DecodeArgs& args, int32_t B, int32_t Hkv, const DecodePlan& pl,
                   hipStream_t st) {
  const unsigned blocks = (unsigned)((int64_t)B * Hkv * pl.splits);
  decode_kernel<D, G, kFp8, kPTH, decode_ring<D, G, kFp8>()><<<blocks, kThreads, 0, st>>>(args);
}

template <int D, int G>
static void dispatch_dtype(const kvq_cache_desc* c, const DecodeArgs& args, int32_t B,
                           const DecodePlan& pl, hipStream_t st) {
  if (c->dtype == KVQ_BF16)
    launch<D, G, false, false>(args, B, c->num_kv_heads, pl, st);
  else if (c->mode == KVQ_SCALE_PER_TOKEN_HEAD)
    launch<D, G, true, true>(args, B, c->num_kv_heads, pl, st);
  else
    launch<D, G, true, false>(args, B, c->num_kv_heads, pl, st);
}

template <int D>
static void dispatch_group(int G, const kvq_cache_desc* c, const DecodeArgs& args, int32_t B,
                           const DecodePlan& pl, hipStream_t st) {
  switch (G) {
    case 1: dispatch_dtype<D, 1>(c, args, B, pl, st); break;
    case 2: dispatch_dtype<D, 2>(c, args, B, pl, st); break;
    case 4: dispatch_dtype<D, 4>(c, args, B, pl, st); break;
    case 8: dispatch_dtype<D, 8>(c, args, B, pl, st); break;
    case 16: dispatch_dtype<D, 16>(c, args, B, pl, st); break;
  }
}

}  // namespace kvq

using namespace kvq;

extern "C" kvq_status kvq_decode_workspace_bytes(const kvq_cache_desc* cache,
                                                 int32_t num_seqs, int32_t num_q_heads,
                                                 int32_t max_seq_len, int32_t window,
                                                 int32_t pages_per_split, size_t* bytes) {
  clear_error();
  if (!bytes) return fail(KVQ_ERR_INVALID_ARG, "bytes is NULL");
  DecodePlan pl;
  if (kvq_status s = plan_decode(cache, num_seqs, num_q_heads, max_seq_len, window,
                                 pages_per_split, &pl))
    return s;
  *bytes = pl.bytes;
  return KVQ_OK;
}

namespace kvq {

// The decode entry points' common body (k_new == nullptr: plain decode).
kvq_status decode_impl(
    const kvq_cache_desc* cache, const void* q, int32_t num_seqs, int32_t num_q_heads,
    const int32_t* block_table, int32_t block_table_stride, const int32_t* seq_lens,
    int32_t max_seq_len, const kvq_scales* scales, int32_t window, float softmax_scale,
    int32_t pages_per_split, void* out, kvq_dtype out_dtype, void* workspace,
    size_t workspace_bytes, void* stream, const void* k_new, const void* v_new) {
  DecodePlan pl;
  if (kvq_status s = plan_decode(cache, num_seqs, num_q_heads, max_seq_len, window,
                                 pages_per_split, &pl))
    return s;
  if (num_seqs == 0) return KVQ_OK;
  if (out_dtype != KVQ_BF16 && out_dtype != KVQ_F32)
    return fail(KVQ_ERR_UNSUPPORTED, "out_dtype %d (bf16 or f32)", (int)out_dtype);
  if (!q || !out || !seq_lens || (max_seq_len > 0 && !block_table))
    return fail(KVQ_ERR_INVALID_ARG, "q, out, seq_lens or block_table is NULL");
  if ((uintptr_t)q & 15u) return fail(KVQ_ERR_INVALID_ARG, "q must be 16-byte aligned");
  const int maxp = max_visible_pages(max_seq_len, 0);
  if (max_seq_len > 0 && block_table_stride < maxp)
    return fail(KVQ_ERR_INVALID_ARG, "block_table_stride %d < pages of max_seq_len %d",
                block_table_stride, maxp);
  if (cache->dtype == KVQ_FP8_E4M3) {
    if (!scales) return fail(KVQ_ERR_INVALID_ARG, "fp8 cache needs scales");
    if (!(scales->q_scale > 0.0f) ||
        (cache->mode == KVQ_SCALE_PER_TENSOR &&
         !(scales->k_scale > 0.0f && scales->v_scale > 0.0f)))
      return fail(KVQ_ERR_INVALID_ARG, "scales must be > 0");
  }
  if (!(softmax_scale >= 0.0f)) return fail(KVQ_ERR_INVALID_ARG, "softmax_scale < 0");
  if (pl.bytes > 0 && (!workspace || workspace_bytes < pl.bytes))
    return fail(KVQ_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes,
                pl.bytes);
  if (pl.bytes > 0 && ((uintptr_t)workspace & 15u))
    return fail(KVQ_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  auto st = static_cast<hipStream_t>(stream);
  const int D = cache->head_dim;
  const int G = num_q_heads / cache->num_kv_heads;
  const float sm = softmax_scale > 0.0f ? softmax_scale : 1.0f / sqrtf((float)D);
  DecodeArgs args;
  args.q = static_cast<const uint16_t*>(q);
  args.num_kv_heads = cache->num_kv_heads;
  args.splits = pl.splits;
  args.pps = pl.pps;
  args.max_len = max_seq_len;
  args.block_table = block_table;
  args.bt_stride = block_table_stride;
  args.seq_lens = seq_lens;
  args.k_pages = static_cast<const uint8_t*>(cache->k_pages);
  args.v_pages = static_cast<const uint8_t*>(cache->v_pages);
  args.k_scales = cache->k_scales;
  args.v_scales = cache->v_scales;
  args.q_scale = scales ? scales->q_scale : 1.0f;
  args.k_scale = scales ? scales->k_scale : 1.0f;
  args.v_scale = scales ? scales->v_scale : 1.0f;
  args.head_scales = cache->dtype == KVQ_FP8_E4M3 && cache->mode == KVQ_SCALE_PER_KV_HEAD;
  args.sm_log2 = sm * kLog2e;
  args.window = window;
  args.counters = pl.bytes ? static_cast<int32_t*>(workspace) : nullptr;
  args.o_part = pl.bytes ? reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                                    kCounterBytes)
                         : nullptr;
  args.ml_part = pl.bytes ? args.o_part + (size_t)num_seqs * num_q_heads * pl.splits * D
                          : nullptr;
  args.out = out;
  args.out_f32 = out_dtype == KVQ_F32;
  args.k_new = static_cast<const uint16_t*>(k_new);
  args.v_new = static_cast<const uint16_t*>(v_new);
  switch (D) {
    case 64: dispatch_group<64>(G, cache, args, num_seqs, pl, st); break;
    case 128: dispatch_group<128>(G, cache, args, num_seqs, pl, st); break;
    case 256: dispatch_group<256>(G, cache, args, num_seqs, pl, st); break;
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  return KVQ_OK;
}

}  // namespace kvq

extern "C" kvq_status kvq_decode_attention(
    const kvq_cache_desc* cache, const void* q, int32_t num_seqs, int32_t num_q_heads,
    const int32_t* block_table, int32_t block_table_stride, const int32_t* seq_lens,
    int32_t max_seq_len, const kvq_scales* scales, int32_t window, float softmax_scale,
    int32_t pages_per_split, void* out, kvq_dtype out_dtype, void* workspace,
    size_t workspace_bytes, void* stream) {
  clear_error();
  return decode_impl(cache, q, num_seqs, num_q_heads, block_table, block_table_stride,
                     seq_lens, max_seq_len, scales, window, softmax_scale, pages_per_split,
                     out, out_dtype, workspace, workspace_bytes, stream, nullptr, nullptr);
}

extern "C" kvq_status kvq_decode_step(
    const kvq_cache_desc* cache, const void* q, const void* k_new, const void* v_new,
    int32_t num_seqs, int32_t num_q_heads, const int32_t* block_table,
    int32_t block_table_stride, const int32_t* seq_lens, int32_t max_seq_len,
    const kvq_scales* scales, int32_t window, float softmax_scale, int32_t pages_per_split,
    void* out, kvq_dtype out_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  if (num_seqs > 0 && (!k_new || !v_new))
    return fail(KVQ_ERR_INVALID_ARG, "k_new or v_new is NULL");
  if (((uintptr_t)k_new | (uintptr_t)v_new) & 15u)
    return fail(KVQ_ERR_INVALID_ARG, "k_new and v_new must be 16-byte aligned");
  return decode_impl(cache, q, num_seqs, num_q_heads, block_table, block_table_stride,
                     seq_lens, max_seq_len, scales, window, softmax_scale, pages_per_split,
                     out, out_dtype, workspace, workspace_bytes, stream, k_new, v_new);
}
