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
// reference row maximum (rescale only when a score exceeds it by 2^8), so the
// weights p stay <= 256.  P' = e4m3(p * v_scale_j / (v_ref * prob_scale)), where
// v_ref is a running maximum of the per-token V scales (per-token-head mode) or
// the per-tensor V scale; folding v_scale_j into P' before rounding lets the FP8
// product carry per-token V scales.  The row sum l accumulates the same rounded
// P' (mapped back by v_ref * prob_scale / v_scale_j), so the output stays a convex
// combination of V rows.
//
// Accumulation.  Level 1 is one MFMA's 64-key (PV) or 64-dim (QK) sum inside the
// matrix core, whose internal alignment is coarser than float32; level 2 is the
// MFMA's float32 C operand, into which every 64-key chunk is added: on gfx950 this
// add matches a separate float32 VALU add of a fresh result (measured over chains
// of up to 640 chunks), so the running output lives in true float32 registers.
#include "kvq_device.h"
#include "kvq_host.h"

namespace kvq {
namespace pf {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kRows = 32;                 // rows per wave
constexpr int kWgRows = kWaves * kRows;   // rows per workgroup
constexpr int kTile = 64;                 // keys per tile (4 pages)
constexpr int kTilePages = kTile / kPage;
constexpr float kSlack = 8.0f;            // log2 units
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kE4m3Max = 448.0f;

__device__ __forceinline__ v16f mfma(v8i a, v8i b, v16f c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// LDS layout of one tile buffer.
//   K:  [64 keys][D bytes], the 16-byte chunks of key k stored at chunk (c ^ k % NC)
//       (XOR swizzle: the 32 lanes reading one chunk column hit distinct banks).
//   VT: [D dims][80 bytes]: per dim, 2 groups x 32 bytes (the key order of the PV
//       contraction, see vt_offset) + 16 bytes of padding against bank conflicts.
//   scales: float c[64] (score multiplier per key), vs[64], inv_vs[64].
template <int D>
struct Layout {
  static constexpr int NC = D / 16;
  static constexpr int K_OFF = 0;
  static constexpr int VT_PITCH = 80;
  static constexpr int VT_OFF = kTile * D;
  static constexpr int SC_OFF = VT_OFF + D * VT_PITCH;
  static constexpr int BYTES = SC_OFF + 3 * kTile * 4;
};

// Key order of the PV contraction.  In the 32x32 MFMA result, lane l (group
// g = l / 32) register r of key block kb holds key 32 kb + 8 (r / 4) + 4 g + r % 4;
// P' packs those bytes in register order, i.e. byte 16 kb + r of the lane's 32-byte
// B operand.  V^T row (d, g) is stored in that order: dword 4 kb + a holds keys
// 32 kb + 8 a + 4 g + 0..3.
__device__ __forceinline__ int vt_dword(int kb, int a) { return 4 * kb + a; }

struct PrefillArgs {
  const uint16_t* q;
  const int32_t* cu_q_lens;
  int32_t num_kv_heads, tiles;
  const int32_t* block_table;
  int32_t bt_stride;
  const int32_t* seq_lens;
  const uint8_t* k_pages;
  const uint8_t* v_pages;
  const float* k_scales;
  const float* v_scales;
  float q_scale, k_scale, v_scale, prob_scale, sm_log2;
  int32_t causal, window;
  void* out;
  int32_t out_f32;
};

template <int D, int G, bool kPTH>
struct Staging {
  static constexpr int KCH = kTile * D / 16 / kThreads;  // K chunks per thread
  static constexpr int VCH = kTilePages * D / kThreads;   // V rows per thread
  uint4 k[KCH];
  uint4 v[VCH];
  float sc;  // threads 0..63: K scale of key tid; 64..127: V scale of key tid - 64
};

template <int D, int G, bool kPTH>
__global__ __launch_bounds__(kThreads) void prefill_kernel(const PrefillArgs a) {
  using LY = Layout<D>;
  using ST = Staging<D, G, kPTH>;
  constexpr int NP = kWgRows / G;  // query positions per workgroup
  constexpr int KS = D / 64;       // 64-dim steps of the QK contraction
  constexpr int DB = D / 32;       // 32-dim blocks of the output
  __shared__ __align__(16) uint8_t lds[2][LY::BYTES];

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
  const int t_first = wg_lo / kTile;
  const int t_last = wg_hi / kTile;
  const int npages = (L + kPage - 1) / kPage;
  const int* bt = a.block_table + (int64_t)b * a.bt_stride;
  // per-wave bounds for the mask decision
  const int w_hi_min = __builtin_amdgcn_readfirstlane(
      a.causal ? ctx + min(p0 + (wave * kRows) / G, n - 1) : L - 1);
  const int w_lo_max = __builtin_amdgcn_readfirstlane(
      a.window > 0 ? max(0, ctx + min(p0 + (wave * kRows + kRows - 1) / G, n - 1) -
                                a.window + 1)
                   : 0);

  // ---- query codes: B operand of S^T = K . Q^T -----------------------------------
  // lane holds row `row`, dims 64 ks + 32 grp + 0..31 as 32 e4m3 codes per step.
  v8i qb[KS];
  {
    const uint16_t* qrow = a.q + ((int64_t)(q0 + min(p_loc, n - 1)) * Hq + g * G + hh) * D;
    const bool unit_q = a.q_scale == 1.0f;
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
            const float f = bf16_bits_to_float(bits);
            const uint32_t code = unit_q ? e4m3_encode(f) : e4m3_quantize(f, a.q_scale);
            word |= (row_ok ? code : 0u) << (8 * e);
          }
          w[2 * c4 + h] = word;
        }
      }
      qb[ks] = (v8i){(int)w[0], (int)w[1], (int)w[2], (int)w[3],
                     (int)w[4], (int)w[5], (int)w[6], (int)w[7]};
    }
  }
  const float qk_base = a.q_scale * a.sm_log2 * (kPTH ? 1.0f : a.k_scale);

  // ---- tile staging: global -> registers -> LDS -----------------------------------
  auto load_tile = [&](int t, ST& s) {
#pragma unroll
    for (int u = 0; u < ST::KCH; ++u) {
      const int c = tid + u * kThreads;
      const int key = c / LY::NC, col = c % LY::NC;
      const int pg = t * kTilePages + key / kPage;
      s.k[u] = make_uint4(0, 0, 0, 0);
      if (pg < npages) {
        const int64_t tileg = (int64_t)bt[pg] * hkv + g;
        s.k[u] = *reinterpret_cast<const uint4*>(
            a.k_pages + (tileg * kPage + key % kPage) * D + col * 16);
      }
    }
#pragma unroll
    for (int u = 0; u < ST::VCH; ++u) {
      const int c = tid + u * kThreads;
      const int pl = c / D, d = c % D;
      const int pg = t * kTilePages + pl;
      s.v[u] = make_uint4(0, 0, 0, 0);
      if (pg < npages) {
        const int64_t tileg = (int64_t)bt[pg] * hkv + g;
        s.v[u] = *reinterpret_cast<const uint4*>(a.v_pages + (tileg * D + d) * kPage);
        // slots past the sequence end were never written: their bytes may be any
        // code, NaN included, and 0 * NaN would poison the product
        const int valid = L - pg * kPage;
        if (valid < kPage) {
          uint32_t w[4] = {s.v[u].x, s.v[u].y, s.v[u].z, s.v[u].w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int keep = min(max(valid - 4 * j, 0), 4);  // bytes kept in word j
            w[j] &= keep >= 4 ? 0xFFFFFFFFu : ((1u << (8 * keep)) - 1u);
          }
          s.v[u] = make_uint4(w[0], w[1], w[2], w[3]);
        }
      }
    }
    s.sc = 0.0f;
    if constexpr (kPTH) {
      if (tid < 2 * kTile) {
        const int key = tid % kTile;
        const int pg = t * kTilePages + key / kPage;
        if (t * kTile + key < L) {
          const int64_t idx = ((int64_t)bt[pg] * hkv + g) * kPage + key % kPage;
          s.sc = tid < kTile ? a.k_scales[idx] : a.v_scales[idx];
        }
      }
    }
  };
  auto store_tile = [&](int t, const ST& s, uint8_t* buf) {
#pragma unroll
    for (int u = 0; u < ST::KCH; ++u) {
      const int c = tid + u * kThreads;
      const int key = c / LY::NC, col = c % LY::NC;
      *reinterpret_cast<uint4*>(buf + LY::K_OFF + key * D + (col ^ (key % LY::NC)) * 16) = s.k[u];
    }
#pragma unroll
    for (int u = 0; u < ST::VCH; ++u) {
      const int c = tid + u * kThreads;
      const int pl = c / D, d = c % D;
      const int kb = pl / 2, a0 = 2 * (pl % 2);
      uint8_t* rowp = buf + LY::VT_OFF + d * LY::VT_PITCH;
      // dwords 0, 2 of the 16-token row belong to group 0, dwords 1, 3 to group 1
      *reinterpret_cast<uint2*>(rowp + 4 * vt_dword(kb, a0)) = make_uint2(s.v[u].x, s.v[u].z);
      *reinterpret_cast<uint2*>(rowp + 32 + 4 * vt_dword(kb, a0)) = make_uint2(s.v[u].y, s.v[u].w);
    }
    float* sc = reinterpret_cast<float*>(buf + LY::SC_OFF);
    if constexpr (kPTH) {
      if (tid < kTile) {
        sc[tid] = s.sc * qk_base;  // score multiplier of key tid
      } else if (tid < 2 * kTile) {
        sc[tid] = s.sc;                                               // v scale
        sc[tid + kTile] = s.sc > 0.0f ? 1.0f / s.sc : 0.0f;           // its inverse
      }
    }
  };

  // ---- running state ---------------------------------------------------------------
  v16f o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = (v16f){};
  float m = -INFINITY;     // reference row maximum (log2 units), same in both lane halves
  float lam = 0.0f;        // this lane's part of the row sum, in P' units / v_scale_j
  float vref = kPTH ? 0.0f : a.v_scale;
  float pmul = kPTH ? 0.0f : 1.0f / a.prob_scale;  // p -> P' factor (times v_scale_j)

  {
    ST s0;
    load_tile(t_first, s0);
    store_tile(t_first, s0, lds[t_first & 1]);
  }
  __syncthreads();

  for (int t = t_first; t <= t_last; ++t) {
    ST s1;
    const bool more = t < t_last;
    if (more) load_tile(t + 1, s1);
    const uint8_t* buf = lds[t & 1];
    const float* sc = reinterpret_cast<const float*>(buf + LY::SC_OFF);

    // ---- running V-scale reference (per-token-head) ------------------------------
    if constexpr (kPTH) {
      float vm = sc[kTile + lane];
      vm = wave_max(vm);
      if (vm > vref) {
        const float f = vref > 0.0f ? vref / vm : 0.0f;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] *= f;
        lam *= f;
        vref = vm;
        pmul = 1.0f / (vref * a.prob_scale);
      }
    }

    // ---- S^T = K . Q^T for the two 32-key blocks --------------------------------
    v16f s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = (v16f){};
      const int key = 32 * kb + row;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int c0 = 4 * ks + 2 * grp;
        const uint4 x0 = *reinterpret_cast<const uint4*>(
            buf + LY::K_OFF + key * D + ((c0) ^ (key % LY::NC)) * 16);
        const uint4 x1 = *reinterpret_cast<const uint4*>(
            buf + LY::K_OFF + key * D + ((c0 + 1) ^ (key % LY::NC)) * 16);
        const v8i ka = {(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                        (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        s[kb] = mfma(ka, qb[ks], s[kb]);
      }
    }

    // ---- scale, mask, lazy rescale -----------------------------------------------
    const int kbase = t * kTile;
    const bool need_mask = (kbase + kTile - 1 > w_hi_min) || (kbase < w_lo_max) ||
                           (kbase + kTile > L);
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int k0 = 32 * kb + 8 * q4 + 4 * grp;  // first of 4 consecutive keys
        float4 c4;
        if constexpr (kPTH) c4 = *reinterpret_cast<const float4*>(sc + k0);
        else c4 = make_float4(qk_base, qk_base, qk_base, qk_base);
        const float cc[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float x = s[kb][4 * q4 + e] * cc[e];
          if (need_mask) {
            const int key = kbase + k0 + e;
            x = (key >= lo && key <= hi && row_ok) ? x : -INFINITY;
          }
          s[kb][4 * q4 + e] = x;
          mx = fmaxf(mx, x);
        }
      }
    if (__builtin_amdgcn_ballot_w64(mx > m + kSlack) != 0) {
      const float rmax = fmaxf(mx, __shfl_xor(mx, kRows));
      const float mn = fmaxf(m, rmax);
      const float alpha = (m == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m - mn);
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
      lam *= alpha;
      m = mn;
    }
    const float msafe = m == -INFINITY ? 0.0f : m;

    // ---- P' (e4m3) in the B-operand layout; row sum from the rounded values -------
    uint32_t pw[8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int k0 = 32 * kb + 8 * q4 + 4 * grp;
        float vs[4] = {1.0f, 1.0f, 1.0f, 1.0f}, ivs[4] = {1.0f, 1.0f, 1.0f, 1.0f};
        if constexpr (kPTH) {
          const float4 v4 = *reinterpret_cast<const float4*>(sc + kTile + k0);
          const float4 i4 = *reinterpret_cast<const float4*>(sc + 2 * kTile + k0);
          vs[0] = v4.x; vs[1] = v4.y; vs[2] = v4.z; vs[3] = v4.w;
          ivs[0] = i4.x; ivs[1] = i4.y; ivs[2] = i4.z; ivs[3] = i4.w;
        }
        float pq[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = __builtin_amdgcn_exp2f(s[kb][4 * q4 + e] - msafe);
          pq[e] = fminf(p * (vs[e] * pmul), kE4m3Max);
        }
        uint32_t word = __builtin_amdgcn_cvt_pk_fp8_f32(pq[0], pq[1], 0, false);
        word = __builtin_amdgcn_cvt_pk_fp8_f32(pq[2], pq[3], word, true);
        pw[4 * kb + q4] = word;
        const float2_t d01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, false);
        const float2_t d23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, true);
        lam = fmaf(d01.x, ivs[0], lam);
        lam = fmaf(d01.y, ivs[1], lam);
        lam = fmaf(d23.x, ivs[2], lam);
        lam = fmaf(d23.y, ivs[3], lam);
      }
    const v8i pb = {(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3],
                    (int)pw[4], (int)pw[5], (int)pw[6], (int)pw[7]};

    // ---- O^T += V^T . P'^T -------------------------------------------------------------
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const uint8_t* vr = buf + LY::VT_OFF + (32 * db + row) * LY::VT_PITCH + 32 * grp;
      const uint4 x0 = *reinterpret_cast<const uint4*>(vr);
      const uint4 x1 = *reinterpret_cast<const uint4*>(vr + 16);
      const v8i va = {(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                      (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
      o[db] = mfma(va, pb, o[db]);
    }

    // The other buffer was last read while computing tile t - 1, which every wave
    // finished before the barrier that ended that iteration.
    if (more) {
      store_tile(t + 1, s1, lds[(t + 1) & 1]);
      __syncthreads();
    }
  }

  // ---- normalise and store: lane holds row `row`, dims 32 db + 8 (r/4) + 4 grp + r%4
  const float lsum = lam + __shfl_xor(lam, kRows);
  // o * (v_ref * prob_scale) / (lsum * v_ref * prob_scale) for per-token-head scales;
  // per-tensor: numerator o * prob_scale * v_scale, row sum lsum * prob_scale
  const float inv = lsum > 0.0f ? (kPTH ? 1.0f : a.v_scale) / lsum : 0.0f;
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

template <int D, int G>
static void launch_mode(const kvq_cache_desc* c, const PrefillArgs& args, unsigned blocks,
                        hipStream_t st) {
  if (c->mode == KVQ_SCALE_PER_TOKEN_HEAD)
    prefill_kernel<D, G, true><<<blocks, kThreads, 0, st>>>(args);
  else
    prefill_kernel<D, G, false><<<blocks, kThreads, 0, st>>>(args);
}

template <int D>
static void launch_group(int G, const kvq_cache_desc* c, const PrefillArgs& args,
                         unsigned blocks, hipStream_t st) {
  switch (G) {
    case 1: launch_mode<D, 1>(c, args, blocks, st); break;
    case 2: launch_mode<D, 2>(c, args, blocks, st); break;
    case 4: launch_mode<D, 4>(c, args, blocks, st); break;
    case 8: launch_mode<D, 8>(c, args, blocks, st); break;
    case 16: launch_mode<D, 16>(c, args, blocks, st); break;
  }
}

}  // namespace pf
}  // namespace kvq

using namespace kvq;

extern "C" kvq_status kvq_prefill_attention(const kvq_cache_desc* cache, const void* q,
                                            const int32_t* cu_q_lens, int32_t num_seqs,
                                            int32_t num_q_heads, const int32_t* block_table,
                                            int32_t block_table_stride, const int32_t* seq_lens,
                                            int32_t max_q_len, const kvq_scales* scales,
                                            int32_t causal, int32_t window, float softmax_scale,
                                            void* out, kvq_dtype out_dtype, void* stream) {
  clear_error();
  if (kvq_status s = check_cache(cache)) return s;
  if (cache->dtype != KVQ_FP8_E4M3)
    return fail(KVQ_ERR_UNSUPPORTED, "prefill reads an fp8 cache (bf16 cache prefill is not built)");
  if (num_seqs < 0 || num_q_heads <= 0 || max_q_len < 0 || window < 0)
    return fail(KVQ_ERR_INVALID_ARG, "num_seqs %d num_q_heads %d max_q_len %d window %d",
                num_seqs, num_q_heads, max_q_len, window);
  if (num_q_heads % cache->num_kv_heads)
    return fail(KVQ_ERR_INVALID_ARG, "num_q_heads %d not a multiple of num_kv_heads %d",
                num_q_heads, cache->num_kv_heads);
  const int G = num_q_heads / cache->num_kv_heads;
  if (!supported_group(G))
    return fail(KVQ_ERR_UNSUPPORTED, "group size %d (1, 2, 4, 8, 16 are built)", G);
  if (num_seqs == 0 || max_q_len == 0) return KVQ_OK;
  if (out_dtype != KVQ_BF16 && out_dtype != KVQ_F32)
    return fail(KVQ_ERR_UNSUPPORTED, "out_dtype %d (bf16 or f32)", (int)out_dtype);
  if (!q || !out || !cu_q_lens || !seq_lens || !block_table)
    return fail(KVQ_ERR_INVALID_ARG, "q, out, cu_q_lens, seq_lens or block_table is NULL");
  if (((uintptr_t)q | (uintptr_t)out) & 15u)
    return fail(KVQ_ERR_INVALID_ARG, "q and out must be 16-byte aligned");
  if (block_table_stride <= 0) return fail(KVQ_ERR_INVALID_ARG, "block_table_stride <= 0");
  if (!scales) return fail(KVQ_ERR_INVALID_ARG, "scales is NULL");
  if (!(scales->q_scale > 0.0f) || !(scales->prob_scale > 0.0f) ||
      (cache->mode == KVQ_SCALE_PER_TENSOR && !(scales->k_scale > 0.0f && scales->v_scale > 0.0f)))
    return fail(KVQ_ERR_INVALID_ARG, "scales must be > 0");
  if (!(softmax_scale >= 0.0f)) return fail(KVQ_ERR_INVALID_ARG, "softmax_scale < 0");
  const int D = cache->head_dim;
  const int np = pf::kWgRows / G;
  pf::PrefillArgs args;
  args.q = static_cast<const uint16_t*>(q);
  args.cu_q_lens = cu_q_lens;
  args.num_kv_heads = cache->num_kv_heads;
  args.tiles = (max_q_len + np - 1) / np;
  args.block_table = block_table;
  args.bt_stride = block_table_stride;
  args.seq_lens = seq_lens;
  args.k_pages = static_cast<const uint8_t*>(cache->k_pages);
  args.v_pages = static_cast<const uint8_t*>(cache->v_pages);
  args.k_scales = cache->k_scales;
  args.v_scales = cache->v_scales;
  args.q_scale = scales->q_scale;
  args.k_scale = scales->k_scale;
  args.v_scale = scales->v_scale;
  args.prob_scale = scales->prob_scale;
  const float sm = softmax_scale > 0.0f ? softmax_scale : 1.0f / sqrtf((float)D);
  args.sm_log2 = sm * pf::kLog2e;
  args.causal = causal != 0;
  args.window = window;
  args.out = out;
  args.out_f32 = out_dtype == KVQ_F32;
  const int64_t blocks = (int64_t)num_seqs * cache->num_kv_heads * args.tiles;
  if (blocks > 0x7FFFFFFF) return fail(KVQ_ERR_INVALID_ARG, "grid too large");
  auto st = static_cast<hipStream_t>(stream);
  switch (D) {
    case 64: pf::launch_group<64>(G, cache, args, (unsigned)blocks, st); break;
    case 128: pf::launch_group<128>(G, cache, args, (unsigned)blocks, st); break;
    case 256: pf::launch_group<256>(G, cache, args, (unsigned)blocks, st); break;
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
  return KVQ_OK;
}
