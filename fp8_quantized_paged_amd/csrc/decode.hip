// Split-K paged GQA decode attention over an FP8 (or bf16) cache, and the merge.
//
// Method: "vLLM FP8 KV-Cache and Attention Quantization Update" (agentlenshq.com):
// FP8 e4m3 storage halves the bytes each decode step reads (section "Performance
// benchmarking"), attention runs on the FP8 values, partial sums are kept in true
// float32 registers (section "Two-level accumulation"), sliding-window layers may
// keep a bf16 cache (section "Hybrid attention and layer skipping"); the query is
// quantised inside the attention op (section "Kernel and fusion optimizations").
//
// Work split.  One wavefront owns one (sequence b, KV head g, split s) and serves
// all G query heads of the group.  A split is a run of at most 64 cache pages of
// the sequence's visible key range; a workgroup holds four independent waves.
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
//         rows of the dim-major V tile (one 16-byte load per channel), converted
//         to float32.  The float32 weights p * v_scale are broadcast through LDS
//         and accumulated with float32 FMAs (weights are not rounded below
//         float32: with outlier channels the sum cancels large terms).
// Accumulation levels: one page inside the dot2 chains / FMA chains, the split in
// float32 registers, splits merged in float32 by the merge kernel.
#include "kvq_device.h"
#include "kvq_host.h"

namespace kvq {

constexpr int ilog2c(int x) { return x <= 1 ? 0 : 1 + ilog2c(x / 2); }
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.0f;  // log2 units: weights stay <= 256
constexpr int kMaxPagesPerSplit = 64;
constexpr int kWavesPerBlock = 4;

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
  static constexpr int Q_WORDS = G * D / 2;         // query (bf16) in LDS
  static constexpr int P_WORDS = G * kPage;         // weights (float32) in LDS
  static constexpr int LDS_WORDS = (kFp8 ? Q_WORDS : 0) + P_WORDS;
};

// Number of pages a split covers and the visible page range of a sequence.
struct SplitRange {
  int lo;      // first visible key
  int pfirst;  // first visible page
  int pend;    // one past the last page
};

__device__ __forceinline__ SplitRange visible_range(int L, int window) {
  SplitRange r;
  r.lo = window > 0 ? max(0, L - window) : 0;
  r.pfirst = r.lo / kPage;
  r.pend = (L + kPage - 1) / kPage;
  return r;
}

__device__ __forceinline__ void store_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float load_agent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_out(void* out, int32_t out_f32, int64_t i, float v) {
  if (out_f32)
    static_cast<float*>(out)[i] = v;
  else
    static_cast<uint16_t*>(out)[i] = (uint16_t)float_to_bf16_bits(v);
}

// Butterfly over lane bits [LOG_LPT-1 .. LOG_LPT-NB] then all-reduce over the rest.
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

template <int NVL, int STEP, int NAR>
__device__ __forceinline__ void allreduce_low_bits(float (&v)[NVL]) {
  if constexpr (STEP < NAR) {
    constexpr int bit = NAR - 1 - STEP;
#pragma unroll
    for (int k = 0; k < NVL; ++k) v[k] += dpp_partner<bit>(v[k]);
    allreduce_low_bits<NVL, STEP + 1, NAR>(v);
  }
}

template <int D, int G, bool kFp8, bool kPTH>
__global__ __launch_bounds__(256) void decode_split_kernel(
    const uint16_t* __restrict__ q, int32_t num_seqs, int32_t num_kv_heads,
    int32_t splits, int32_t pps, const int32_t* __restrict__ block_table,
    int32_t bt_stride, const int32_t* __restrict__ seq_lens,
    const uint8_t* __restrict__ k_pages, const uint8_t* __restrict__ v_pages,
    const float* __restrict__ k_scales, const float* __restrict__ v_scales,
    float q_scale, float k_scale, float v_scale, float sm_log2, int32_t window,
    float* __restrict__ o_part, float* __restrict__ ml_part, int32_t* __restrict__ counters,
    void* __restrict__ out, int32_t out_f32) {
  using S = DecodeShape<D, G, kFp8>;
  __shared__ uint32_t lds_all[kWavesPerBlock][S::LDS_WORDS];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int64_t w = (int64_t)blockIdx.x * kWavesPerBlock + wave;
  if (w >= (int64_t)num_seqs * num_kv_heads * splits) return;
  const int s = (int)(w % splits);
  const int g = (int)((w / splits) % num_kv_heads);
  const int b = (int)(w / ((int64_t)splits * num_kv_heads));
  const int L = seq_lens[b];
  const SplitRange vr = visible_range(L, window);
  const int pb = vr.pfirst + s * pps;
  const int pe = min(pb + pps, vr.pend);
  const int ns = L > 0 ? (vr.pend - vr.pfirst + pps - 1) / pps : 0;  // splits of (b, g)
  const int num_q_heads = num_kv_heads * G;
  if (s >= ns) {
    if (s == 0) {  // empty sequence: zero output rows
      for (int e = lane; e < G * D; e += kWave)
        store_out(out, out_f32, ((int64_t)b * num_q_heads + g * G) * D + e, 0.0f);
    }
    return;
  }

  uint32_t* lds = lds_all[wave];
  uint32_t* p_lds = lds + (kFp8 ? S::Q_WORDS : 0);
  const int tg = lane / S::LPT;   // token group (QK layout)
  const int c = lane % S::LPT;    // channel chunk: channels 16c .. 16c+15

  // ---- query: fused e4m3 quantisation (fp8) or plain bf16 -----------------------
  const uint16_t* qg = q + ((int64_t)b * num_q_heads + (int64_t)g * G) * D;
  uint32_t qv[G][8];  // bf16 pairs of channels 16c .. 16c+15, per head
  if constexpr (kFp8) {
    const bool unit_q = q_scale == 1.0f;
    for (int e = lane * 8; e < G * D; e += kWave * 8) {
      const uint4 x = *reinterpret_cast<const uint4*>(qg + e);
      const uint32_t xx[4] = {x.x, x.y, x.z, x.w};
      uint32_t out[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // x / 1.0 == x exactly, so the division is skipped for a unit scale
        const float x0 = bf16_bits_to_float(xx[i] & 0xFFFFu);
        const float x1 = bf16_bits_to_float(xx[i] >> 16);
        const uint32_t c0 = unit_q ? e4m3_encode(x0) : e4m3_quantize(x0, q_scale);
        const uint32_t c1 = unit_q ? e4m3_encode(x1) : e4m3_quantize(x1, q_scale);
        out[i] = __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2<false>(c0 | (c1 << 8)));
      }
      *reinterpret_cast<uint4*>(lds + e / 2) = make_uint4(out[0], out[1], out[2], out[3]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const uint4 a = *reinterpret_cast<const uint4*>(lds + (hh * D + c * 16) / 2);
      const uint4 bq = *reinterpret_cast<const uint4*>(lds + (hh * D + c * 16) / 2 + 4);
      qv[hh][0] = a.x; qv[hh][1] = a.y; qv[hh][2] = a.z; qv[hh][3] = a.w;
      qv[hh][4] = bq.x; qv[hh][5] = bq.y; qv[hh][6] = bq.z; qv[hh][7] = bq.w;
    }
  } else {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const uint4* src = reinterpret_cast<const uint4*>(qg + hh * D + c * 16);
      const uint4 a = src[0], bq = src[1];
      qv[hh][0] = a.x; qv[hh][1] = a.y; qv[hh][2] = a.z; qv[hh][3] = a.w;
      qv[hh][4] = bq.x; qv[hh][5] = bq.y; qv[hh][6] = bq.z; qv[hh][7] = bq.w;
    }
  }

  // score multiplier (log2 domain); per-token K scales multiply in per page
  const float qk_base = kFp8 ? q_scale * sm_log2 * (kPTH ? 1.0f : k_scale) : sm_log2;

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

  float m_all[G];
  float m_mine[S::NVL], l_mine[S::NVL];
  float acc[G][S::DPL];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    m_all[hh] = -INFINITY;
#pragma unroll
    for (int dd = 0; dd < S::DPL; ++dd) acc[hh][dd] = 0.0f;
  }
#pragma unroll
  for (int k = 0; k < S::NVL; ++k) {
    m_mine[k] = -INFINITY;
    l_mine[k] = 0.0f;
  }

  const int* bt = block_table + (int64_t)b * bt_stride;
  const int bt_lane = (pb + lane < pe) ? bt[pb + lane] : 0;

  // One page's inputs for this lane: K rows of its token slots, V rows of its
  // channels, and the per-token scales of the scores it will hold.
  struct PageRegs {
    uint32_t kr[S::NT][S::KW];
    uint32_t vrw[S::DPL][S::VW];
    float ksc[S::NVL], vsc[S::NVL];
  };

  auto load_page = [&](int i, PageRegs& r) {
    const int page = __builtin_amdgcn_readlane(bt_lane, i - pb);
    const int64_t tile = (int64_t)page * num_kv_heads + g;
#pragma unroll
    for (int ts = 0; ts < S::NT; ++ts) {
      const int t = tg + ts * S::TPL;
      const uint4* src = reinterpret_cast<const uint4*>(
          k_pages + ((tile * kPage + t) * D + c * 16) * S::EB);
#pragma unroll
      for (int j = 0; j < S::KW / 4; ++j) {
        const uint4 x = src[j];
        r.kr[ts][4 * j] = x.x; r.kr[ts][4 * j + 1] = x.y;
        r.kr[ts][4 * j + 2] = x.z; r.kr[ts][4 * j + 3] = x.w;
      }
    }
#pragma unroll
    for (int dd = 0; dd < S::DPL; ++dd) {
      const uint4* src = reinterpret_cast<const uint4*>(
          v_pages + ((tile * D + lane + kWave * dd) * kPage) * S::EB);
#pragma unroll
      for (int j = 0; j < S::VW / 4; ++j) {
        const uint4 x = src[j];
        r.vrw[dd][4 * j] = x.x; r.vrw[dd][4 * j + 1] = x.y;
        r.vrw[dd][4 * j + 2] = x.z; r.vrw[dd][4 * j + 3] = x.w;
      }
    }
#pragma unroll
    for (int k = 0; k < S::NVL; ++k) {
      if constexpr (kFp8 && kPTH) {
        r.ksc[k] = k_scales[tile * kPage + t_of[k]];
        r.vsc[k] = v_scales[tile * kPage + t_of[k]];
      } else {
        r.ksc[k] = 1.0f;
        r.vsc[k] = kFp8 ? v_scale : 1.0f;
      }
    }
  };

  auto compute_page = [&](int i, const PageRegs& r) {
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
        float a = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) a = dot2_bf16(as_bf16x2(qv[hh][j]), kp[j], a);
        part[ts * G + hh] = a;
      }
    }
    butterfly<S::NV, S::LOG_LPT, S::NB, 0>(part, c);
    float sc[S::NVL];
#pragma unroll
    for (int k = 0; k < S::NVL; ++k) sc[k] = part[k];
    allreduce_low_bits<S::NVL, 0, S::NAR>(sc);

    // ---- scale, mask, lazy rescale ---------------------------------------------
    bool over = false;
#pragma unroll
    for (int k = 0; k < S::NVL; ++k) {
      const int pos = i * kPage + t_of[k];
      sc[k] = (pos >= vr.lo && pos < L) ? sc[k] * (qk_base * r.ksc[k]) : -INFINITY;
      over |= sc[k] > m_mine[k] + kRescaleSlack;
    }
    if (__builtin_amdgcn_ballot_w64(over) != 0) {
      float alpha[G];
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float x = -INFINITY;
#pragma unroll
        for (int k = 0; k < S::NVL; ++k) x = hh_of[k] == hh ? fmaxf(x, sc[k]) : x;
        const float mx = wave_max(x);
        const float mn = fmaxf(m_all[hh], mx);
        alpha[hh] = mn == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_all[hh] - mn);
        m_all[hh] = mn;
#pragma unroll
        for (int dd = 0; dd < S::DPL; ++dd) acc[hh][dd] *= alpha[hh];
      }
#pragma unroll
      for (int k = 0; k < S::NVL; ++k) {
        float a = alpha[0], m = m_all[0];
#pragma unroll
        for (int hh = 1; hh < G; ++hh) {
          a = hh_of[k] == hh ? alpha[hh] : a;
          m = hh_of[k] == hh ? m_all[hh] : m;
        }
        l_mine[k] *= a;
        m_mine[k] = m;
      }
    }

    // ---- weights -> LDS --------------------------------------------------------
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    float* pf = reinterpret_cast<float*>(p_lds);
#pragma unroll
    for (int k = 0; k < S::NVL; ++k) {
      const float p = __builtin_amdgcn_exp2f(sc[k] - m_mine[k]);
      if (owner) {
        l_mine[k] += p;
        pf[hh_of[k] * kPage + t_of[k]] = p * r.vsc[k];
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- PV ----------------------------------------------------------------------
    float vf[S::DPL][kPage];
#pragma unroll
    for (int dd = 0; dd < S::DPL; ++dd)
#pragma unroll
      for (int j = 0; j < kPage / 2; ++j) {
        if constexpr (kFp8) {
          const float2_t f = (j & 1) ? e4m3x2_to_f32x2<true>(r.vrw[dd][j / 2])
                                     : e4m3x2_to_f32x2<false>(r.vrw[dd][j / 2]);
          vf[dd][2 * j] = f.x;
          vf[dd][2 * j + 1] = f.y;
        } else {
          vf[dd][2 * j] = bf16_bits_to_float(r.vrw[dd][j] & 0xFFFFu);
          vf[dd][2 * j + 1] = bf16_bits_to_float(r.vrw[dd][j] >> 16);
        }
      }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float pw[kPage];
#pragma unroll
      for (int j = 0; j < kPage / 4; ++j) {
        const float4 a = *reinterpret_cast<const float4*>(p_lds + hh * kPage + 4 * j);
        pw[4 * j] = a.x; pw[4 * j + 1] = a.y; pw[4 * j + 2] = a.z; pw[4 * j + 3] = a.w;
      }
#pragma unroll
      for (int dd = 0; dd < S::DPL; ++dd) {
        float x = acc[hh][dd];
#pragma unroll
        for (int t = 0; t < kPage; ++t) x = fmaf(pw[t], vf[dd][t], x);
        acc[hh][dd] = x;
      }
    }
  };

  // Ring of three page buffers, written out so every buffer is a named register
  // set: two pages are in flight while the third is computed.
  PageRegs ra, rb, rc;
  load_page(pb, ra);
  if (pb + 1 < pe) load_page(pb + 1, rb);
  for (int i = pb; i < pe; i += 3) {
    if (i + 2 < pe) load_page(i + 2, rc);
    compute_page(i, ra);
    if (i + 1 >= pe) break;
    if (i + 3 < pe) load_page(i + 3, ra);
    compute_page(i + 1, rb);
    if (i + 2 >= pe) break;
    if (i + 4 < pe) load_page(i + 4, rb);
    compute_page(i + 2, rc);
  }

  // ---- split results --------------------------------------------------------------
  float lh[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    float x = 0.0f;
#pragma unroll
    for (int k = 0; k < S::NVL; ++k) x += (owner && hh_of[k] == hh) ? l_mine[k] : 0.0f;
    lh[hh] = wave_sum(x);
  }
  const int64_t out_row0 = (int64_t)b * num_q_heads + g * G;
  if (ns == 1) {  // the only split: normalise and store directly
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float inv = lh[hh] > 0.0f ? 1.0f / lh[hh] : 0.0f;
#pragma unroll
      for (int dd = 0; dd < S::DPL; ++dd)
        store_out(out, out_f32, (out_row0 + hh) * D + lane + kWave * dd, acc[hh][dd] * inv);
    }
    return;
  }
  // partials: o (unnormalised), m (log2 domain), l.  Stored as agent-scope atomics,
  // i.e. written through to the device coherence point (the L2 of each XCD is not
  // coherent with the others), so no L2 write-back is needed to publish them.
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const int64_t row = (out_row0 + hh) * splits + s;
    if (lane == 0) {
      store_agent(&ml_part[row * 2], m_all[hh]);
      store_agent(&ml_part[row * 2 + 1], lh[hh]);
    }
#pragma unroll
    for (int dd = 0; dd < S::DPL; ++dd)  // lane-major: this lane's channels adjacent
      store_agent(&o_part[row * D + lane * S::DPL + dd], acc[hh][dd]);
  }
  // The last split of (b, g) to finish merges all of them (level 3 of the float32
  // accumulation): wait until this wave's partials are performed, then count; the
  // wave that completes the count reads the partials back with agent-scope loads
  // and resets the counter for the next call.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");  // s_waitcnt vmcnt(0)
  int done = 0;
  if (lane == 0)
    done = __hip_atomic_fetch_add(&counters[(int64_t)b * num_kv_heads + g], 1,
                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  done = __builtin_amdgcn_readfirstlane(done);
  if (done != ns - 1) return;
  // Merge with many loads in flight: weights of up to 64 splits sit one per lane;
  // partial rows are fetched kMergeBatch splits x G heads at a time.
  constexpr int kMergeBatch = (G * S::DPL) >= 64 ? 1 : 64 / (G * S::DPL);
  float M[G], lpart[G], o[G][S::DPL];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const int64_t row0 = (out_row0 + hh) * splits;
    float mj = -INFINITY;
    for (int j = lane; j < ns; j += kWave) mj = fmaxf(mj, load_agent(&ml_part[(row0 + j) * 2]));
    M[hh] = wave_max(mj);
    lpart[hh] = 0.0f;
#pragma unroll
    for (int dd = 0; dd < S::DPL; ++dd) o[hh][dd] = 0.0f;
  }
  for (int j0 = 0; j0 < ns; j0 += kWave) {
    float w[G];  // lane x: weight of split j0 + x
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const int64_t row = (out_row0 + hh) * splits + j0 + lane;
      w[hh] = 0.0f;
      if (j0 + lane < ns) {
        const float m = load_agent(&ml_part[row * 2]);
        w[hh] = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - M[hh]);
        lpart[hh] += load_agent(&ml_part[row * 2 + 1]) * w[hh];
      }
    }
    const int cnt = min(kWave, ns - j0);
    for (int x0 = 0; x0 < cnt; x0 += kMergeBatch) {
      float v[G][kMergeBatch][S::DPL];
#pragma unroll
      for (int hh = 0; hh < G; ++hh)
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) {
          const int x = min(x0 + u, cnt - 1);  // clamped rows get weight 0 below
          const int64_t row = (out_row0 + hh) * splits + j0 + x;
#pragma unroll
          for (int dd = 0; dd < S::DPL; ++dd)
            v[hh][u][dd] = load_agent(&o_part[row * D + lane * S::DPL + dd]);
        }
#pragma unroll
      for (int hh = 0; hh < G; ++hh)
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) {
          const float wx = x0 + u < cnt ? __int_as_float(__builtin_amdgcn_readlane(
                                              __float_as_int(w[hh]), x0 + u))
                                        : 0.0f;
#pragma unroll
          for (int dd = 0; dd < S::DPL; ++dd) o[hh][dd] += v[hh][u][dd] * wx;
        }
    }
  }
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const float lsum = wave_sum(lpart[hh]);
    const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
#pragma unroll
    for (int dd = 0; dd < S::DPL; ++dd)
      store_out(out, out_f32, (out_row0 + hh) * D + lane + kWave * dd, o[hh][dd] * inv);
  }
  if (lane == 0)
    __hip_atomic_store(&counters[(int64_t)b * num_kv_heads + g], 0, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// ---- host side ----------------------------------------------------------------------

static int max_visible_pages(int32_t max_seq_len, int32_t window) {
  const int all = (max_seq_len + kPage - 1) / kPage;
  if (window <= 0) return all;
  const int win = (window + kPage - 1) / kPage + 1;
  return all < win ? all : win;
}

// Pages per split: enough splits to put ~16 waves on each of the 256 CUs, each
// split between 4 and 64 pages.
static int auto_pages_per_split(int32_t num_seqs, int32_t num_kv_heads, int max_pages) {
  const int64_t units = (int64_t)num_seqs * num_kv_heads;
  if (units <= 0 || max_pages <= 0) return 4;
  const int64_t target_waves = 256 * 16;
  int64_t splits = (target_waves + units - 1) / units;
  if (splits < 1) splits = 1;
  int64_t pps = (max_pages + splits - 1) / splits;
  if (pps < 4) pps = 4;
  if (pps > kMaxPagesPerSplit) pps = kMaxPagesPerSplit;
  return (int)pps;
}

struct DecodePlan {
  int pps;
  int splits;
  size_t counter_bytes;  // completion counters, int32 [B][Hkv], 256-byte padded
  size_t bytes;
};

static size_t counter_area_bytes(int32_t num_seqs, int32_t num_kv_heads) {
  const size_t n = (size_t)num_seqs * num_kv_heads * sizeof(int32_t);
  return (n + 255) / 256 * 256;
}

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
  plan->counter_bytes = counter_area_bytes(num_seqs, cache->num_kv_heads);
  plan->bytes = plan->counter_bytes + (size_t)num_seqs * num_q_heads * plan->splits *
                                          (cache->head_dim + 2) * sizeof(float);
  return KVQ_OK;
}

template <int D, int G, bool kFp8, bool kPTH>
static void launch_split(const kvq_cache_desc* c, const void* q, int32_t B,
                         const DecodePlan& pl, const int32_t* bt, int32_t bts,
                         const int32_t* sl, const kvq_scales* sc, float sm_log2,
                         int32_t window, float* o_part, float* ml_part, int32_t* counters,
                         void* out, int32_t out_f32, hipStream_t st) {
  const int64_t waves = (int64_t)B * c->num_kv_heads * pl.splits;
  const unsigned blocks = (unsigned)((waves + kWavesPerBlock - 1) / kWavesPerBlock);
  decode_split_kernel<D, G, kFp8, kPTH><<<blocks, 256, 0, st>>>(
      static_cast<const uint16_t*>(q), B, c->num_kv_heads, pl.splits, pl.pps, bt, bts, sl,
      static_cast<const uint8_t*>(c->k_pages), static_cast<const uint8_t*>(c->v_pages),
      c->k_scales, c->v_scales, sc ? sc->q_scale : 1.f, sc ? sc->k_scale : 1.f,
      sc ? sc->v_scale : 1.f, sm_log2, window, o_part, ml_part, counters, out, out_f32);
}

template <int D, int G>
static void dispatch_dtype(const kvq_cache_desc* c, const void* q, int32_t B,
                           const DecodePlan& pl, const int32_t* bt, int32_t bts,
                           const int32_t* sl, const kvq_scales* sc, float sm_log2,
                           int32_t window, float* o, float* ml, int32_t* cnt, void* out,
                           int32_t f32, hipStream_t st) {
  if (c->dtype == KVQ_BF16)
    launch_split<D, G, false, false>(c, q, B, pl, bt, bts, sl, sc, sm_log2, window, o, ml, cnt, out, f32, st);
  else if (c->mode == KVQ_SCALE_PER_TOKEN_HEAD)
    launch_split<D, G, true, true>(c, q, B, pl, bt, bts, sl, sc, sm_log2, window, o, ml, cnt, out, f32, st);
  else
    launch_split<D, G, true, false>(c, q, B, pl, bt, bts, sl, sc, sm_log2, window, o, ml, cnt, out, f32, st);
}

template <int D>
static void dispatch_group(int G, const kvq_cache_desc* c, const void* q, int32_t B,
                           const DecodePlan& pl, const int32_t* bt, int32_t bts,
                           const int32_t* sl, const kvq_scales* sc, float sm_log2,
                           int32_t window, float* o, float* ml, int32_t* cnt, void* out,
                           int32_t f32, hipStream_t st) {
  switch (G) {
    case 1: dispatch_dtype<D, 1>(c, q, B, pl, bt, bts, sl, sc, sm_log2, window, o, ml, cnt, out, f32, st); break;
    case 2: dispatch_dtype<D, 2>(c, q, B, pl, bt, bts, sl, sc, sm_log2, window, o, ml, cnt, out, f32, st); break;
    case 4: dispatch_dtype<D, 4>(c, q, B, pl, bt, bts, sl, sc, sm_log2, window, o, ml, cnt, out, f32, st); break;
    case 8: dispatch_dtype<D, 8>(c, q, B, pl, bt, bts, sl, sc, sm_log2, window, o, ml, cnt, out, f32, st); break;
    case 16: dispatch_dtype<D, 16>(c, q, B, pl, bt, bts, sl, sc, sm_log2, window, o, ml, cnt, out, f32, st); break;
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

extern "C" kvq_status kvq_decode_attention(
    const kvq_cache_desc* cache, const void* q, int32_t num_seqs, int32_t num_q_heads,
    const int32_t* block_table, int32_t block_table_stride, const int32_t* seq_lens,
    int32_t max_seq_len, const kvq_scales* scales, int32_t window, float softmax_scale,
    int32_t pages_per_split, void* out, kvq_dtype out_dtype, void* workspace,
    size_t workspace_bytes, void* stream) {
  clear_error();
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
  const int D = cache->head_dim;
  const int G = num_q_heads / cache->num_kv_heads;
  const float sm = softmax_scale > 0.0f ? softmax_scale : 1.0f / sqrtf((float)D);
  const float sm_log2 = sm * kLog2e;
  int32_t* counters = static_cast<int32_t*>(workspace);
  float* o_part = reinterpret_cast<float*>(static_cast<char*>(workspace) + pl.counter_bytes);
  float* ml_part = o_part + (size_t)num_seqs * num_q_heads * pl.splits * D;
  const int f32 = out_dtype == KVQ_F32;
  auto st = static_cast<hipStream_t>(stream);
  switch (D) {
    case 64: dispatch_group<64>(G, cache, q, num_seqs, pl, block_table, block_table_stride, seq_lens, scales, sm_log2, window, o_part, ml_part, counters, out, f32, st); break;
    case 128: dispatch_group<128>(G, cache, q, num_seqs, pl, block_table, block_table_stride, seq_lens, scales, sm_log2, window, o_part, ml_part, counters, out, f32, st); break;
    case 256: dispatch_group<256>(G, cache, q, num_seqs, pl, block_table, block_table_stride, seq_lens, scales, sm_log2, window, o_part, ml_part, counters, out, f32, st); break;
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  return KVQ_OK;
}
