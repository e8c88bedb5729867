// Chunked prefill over a bf16 cache: the prefill of the sliding-window layers that
// keep bf16 caches ("vLLM FP8 KV-Cache and Attention Quantization Update", section
// "Hybrid attention and layer skipping": those layers skip FP8 and stay in BF16).
//
// Arithmetic: S = Q . K^T on bf16 matrix cores (v_mfma_f32_32x32x16_bf16: exact
// products, float32 sums), float32 online softmax in the log2 domain, the weights
// rounded to bf16 for P . V on the same matrix cores into float32 accumulators, and
// normalisation by the sum of the rounded weights (so the output is an exact convex
// combination of V rows with the rounded weights).
//
// Work split: a workgroup of 4 waves per (sequence, query head, 128 query positions);
// a wave owns 32 positions of one query head and walks the keys they see in tiles of
// 32 (two cache pages).  Per tile, S^T = K . Q^T is one 32x32 accumulator: lane l
// supplies key row l % 32 of K and query column l % 32 of Q^T, and receives query
// l % 32's scores of keys 8 (r / 4) + 4 (l / 32) + r % 4 (register r).  The first
// eight of those keys are exactly the lane's part of the B operand of the first
// 16-key P . V step, the last eight of the second, so the weights never leave the
// lane; V^T rows (channels) come from the dim-major tile, two 8-byte reads per step.
// Sliding-window layers see at most window + 31 keys per wave, so the kernel favours
// plainness over the fp8 kernel's LDS pipeline: a wave reads its page ids 64 at a time
// and keeps the next tile's K and V rows in flight in registers while it computes one.
#include "kvq_device.h"
#include "kvq_host.h"
#include "prefill_bf16.h"

namespace kvq {
namespace pfb {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kRows = 32;               // query positions per wave
constexpr int kWgRows = kWaves * kRows;  // per workgroup

// Waves per SIMD: the launch has many small workgroups whose time is mostly memory
// latency; the register budget this leaves must still hold two tiles in flight.
template <int D>
constexpr int prefill_bf16_waves() { return D == 64 ? 3 : 1; }

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(
    prefill_bf16_waves<D>()))) void prefill_bf16_kernel(const PrefillBf16Args a) {
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
  const int lane = (int)threadIdx.x % kWave;
  const int h = (int)(blockIdx.x % (unsigned)a.num_q_heads);
  const int rest = (int)(blockIdx.x / (unsigned)a.num_q_heads);
  const int tile = rest % a.tiles;
  const int b = rest / a.tiles;
  const int g = h / (a.num_q_heads / a.num_kv_heads);

  const int q0 = a.cu_q_lens[b];
  const int n = a.cu_q_lens[b + 1] - q0;  // new queries of the sequence
  const int L = a.seq_lens[b];
  const int ctx = L - n;
  const int p0 = tile * kWgRows + wave * kRows;  // this wave's first local position
  if (p0 >= n || L <= 0) return;                 // no workgroup barriers below

  const int col = lane % 32;   // query column of S^T, key row of K, channel of V^T
  const int hg = lane / 32;    // lane group: which 8 of each 16-deep contraction step
  const bool row_ok = p0 + col < n;
  const int p = min(p0 + col, n - 1);
  const int qpos = ctx + p;
  const int hi_row = a.causal ? qpos : L - 1;
  const int lo_row = a.window > 0 ? max(0, qpos - a.window + 1) : 0;
  const int w_hi = a.causal ? ctx + min(p0 + kRows - 1, n - 1) : L - 1;
  const int w_lo = a.window > 0 ? max(0, ctx + p0 - a.window + 1) : 0;
  const int t_first = w_lo / 32, t_last = w_hi / 32;
  const int* bt = a.block_table + (int64_t)b * a.bt_stride;
  const int64_t H = a.num_kv_heads;

  // Q^T operand: query column `col`, channels 16 st + 8 hg .. + 7 of step st
  bf16x8_t qb[D / 16];
  {
    const uint16_t* qrow = a.q + ((int64_t)(q0 + p) * a.num_q_heads + h) * D;
#pragma unroll
    for (int st = 0; st < D / 16; ++st)
      qb[st] = *reinterpret_cast<const bf16x8_t*>(qrow + 16 * st + 8 * hg);
  }

  v16f o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = (v16f){};
  float m = -INFINITY;  // running maximum of the query's scores (log2 units)
  float l = 0.0f;       // this lane's part of the sum of the rounded weights

  // Page ids of the wave's tiles, one per lane (page 2 (t - pid_t0) + j of the chunk in
  // lane j: 32 tiles per chunk), and the tiles' K and V rows in two register buffers:
  // the next tile's loads are issued before the current tile is computed, so the
  // block-table -> rows chain is paid once per chunk, not once per tile.
  const int npages = (L + kPage - 1) / kPage;
  int pid = 0, pid_t0 = t_first;
  auto load_pids = [&](int tc) {
    pid = bt[min(2 * tc + lane, npages - 1)];
    pid_t0 = tc;
  };
  load_pids(t_first);
  struct TileRegs {
    bf16x8_t k[D / 16];
    uint2 vlo[2][D / 32], vhi[2][D / 32];
  };
  auto load_tile = [&](int t, TileRegs& r) {
    if (t - pid_t0 >= 32) load_pids(t);  // wave-uniform
    const int pa = __builtin_amdgcn_readlane(pid, 2 * (t - pid_t0));
    const int pb = __builtin_amdgcn_readlane(pid, 2 * (t - pid_t0) + 1);
    const int key = min(t * 32 + col, L - 1);  // keys past the end are masked later
    const int pk = key / kPage == 2 * t ? pa : pb;
    const uint16_t* krow = a.k_pages + (((int64_t)pk * H + g) * kPage + key % kPage) * D;
#pragma unroll
    for (int st = 0; st < D / 16; ++st)
      r.k[st] = *reinterpret_cast<const bf16x8_t*>(krow + 16 * st + 8 * hg);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      if (t * 32 + 16 * c >= L) continue;  // wave-uniform; that page is not used
      const int64_t vt = ((int64_t)(c ? pb : pa) * H + g) * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        // channel 32 db + col: tokens 4 hg .. 4 hg + 3 and 8 + 4 hg .. 8 + 4 hg + 3
        const uint16_t* vrow = a.v_pages + (vt + 32 * db + col) * kPage;
        r.vlo[c][db] = *reinterpret_cast<const uint2*>(vrow + 4 * hg);
        r.vhi[c][db] = *reinterpret_cast<const uint2*>(vrow + 8 + 4 * hg);
      }
    }
  };
  auto compute = [&](int t, const TileRegs& r) {
    // ---- S^T = K . Q^T ------------------------------------------------------------
    v16f s = (v16f){};
#pragma unroll
    for (int st = 0; st < D / 16; ++st) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r.k[st], qb[st], s, 0, 0, 0);
    // ---- mask, online softmax (the query's 32 keys sit in lanes col and col + 32) --
    float x[16];
    float mx = -INFINITY;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int kr = t * 32 + 8 * (rr / 4) + 4 * hg + rr % 4;
      const bool vis = kr >= lo_row && kr <= hi_row && kr < L;
      x[rr] = vis ? s[rr] * a.sm_log2 : -INFINITY;
      mx = fmaxf(mx, x[rr]);
    }
    mx = max_xor<32>(mx);
    const float mn = fmaxf(m, mx);
    const float msafe = mn == -INFINITY ? 0.0f : mn;  // nothing visible yet: all zero
    const float alpha = __builtin_amdgcn_exp2f(m - msafe);  // m = -inf -> 0
    m = mn;
    l *= alpha;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
    bf16x8_t pbw[2];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const __bf16 w = (__bf16)__builtin_amdgcn_exp2f(x[rr] - msafe);
      pbw[rr / 8][rr % 8] = w;
      l += (float)w;
    }
    // ---- O^T += V^T . P^T, one 16-key step per page of the tile -------------------
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int k0 = t * 32 + 16 * c;  // first key of the page (wave-uniform)
      if (k0 >= L) continue;
      const int valid = L - k0;        // written tokens of the page
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        uint2 lo = r.vlo[c][db], hi = r.vhi[c][db];
        if (valid < kPage) {  // unwritten slots may hold NaN: zero them
          const int t0 = 4 * hg, t1 = 8 + 4 * hg;
          lo.x = t0 + 0 < valid ? (t0 + 1 < valid ? lo.x : lo.x & 0xFFFFu) : 0u;
          lo.y = t0 + 2 < valid ? (t0 + 3 < valid ? lo.y : lo.y & 0xFFFFu) : 0u;
          hi.x = t1 + 0 < valid ? (t1 + 1 < valid ? hi.x : hi.x & 0xFFFFu) : 0u;
          hi.y = t1 + 2 < valid ? (t1 + 3 < valid ? hi.y : hi.y & 0xFFFFu) : 0u;
        }
        const uint4 w4 = make_uint4(lo.x, lo.y, hi.x, hi.y);
        const bf16x8_t va = __builtin_bit_cast(bf16x8_t, w4);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pbw[c], o[db], 0, 0, 0);
      }
    }
  };
  if constexpr (D == 64) {
    TileRegs ta, tb;
    load_tile(t_first, ta);
    for (int t = t_first; t <= t_last; t += 2) {
      if (t + 1 <= t_last) load_tile(t + 1, tb);
      compute(t, ta);
      if (t + 1 > t_last) break;
      if (t + 2 <= t_last) load_tile(t + 2, ta);
      compute(t + 1, tb);
    }
  } else {
    // head_dim 128 and 256: one tile at a time, its V rows read after the scores (two
    // tiles in flight, or K and V together, left too few registers: 107 -> 142-170 us
    // at head_dim 128)
      for (int t = t_first; t <= t_last; ++t) {
        // ---- S^T = K . Q^T ------------------------------------------------------------
        const int key = min(t * 32 + col, L - 1);  // keys past the end are masked below
        const uint16_t* krow =
            a.k_pages + (((int64_t)bt[key / kPage] * H + g) * kPage + key % kPage) * D;
        v16f s = (v16f){};
    #pragma unroll
        for (int st = 0; st < D / 16; ++st) {
          const bf16x8_t ka = *reinterpret_cast<const bf16x8_t*>(krow + 16 * st + 8 * hg);
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qb[st], s, 0, 0, 0);
        }
        // ---- mask, online softmax (the query's 32 keys sit in lanes col and col + 32) --
        float x[16];
        float mx = -INFINITY;
    #pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kr = t * 32 + 8 * (r / 4) + 4 * hg + r % 4;
          const bool vis = kr >= lo_row && kr <= hi_row && kr < L;
          x[r] = vis ? s[r] * a.sm_log2 : -INFINITY;
          mx = fmaxf(mx, x[r]);
        }
        mx = max_xor<32>(mx);
        const float mn = fmaxf(m, mx);
        const float msafe = mn == -INFINITY ? 0.0f : mn;  // nothing visible yet: all zero
        const float alpha = __builtin_amdgcn_exp2f(m - msafe);  // m = -inf -> 0
        m = mn;
        l *= alpha;
    #pragma unroll
        for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
        bf16x8_t pb[2];
    #pragma unroll
        for (int r = 0; r < 16; ++r) {
          const __bf16 w = (__bf16)__builtin_amdgcn_exp2f(x[r] - msafe);
          pb[r / 8][r % 8] = w;
          l += (float)w;
        }
        // ---- O^T += V^T . P^T, one 16-key step per page of the tile -------------------
    #pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int k0 = t * 32 + 16 * c;  // first key of the page (wave-uniform)
          if (k0 >= L) continue;
          const int valid = L - k0;        // written tokens of the page
          const int64_t vt = ((int64_t)bt[k0 / kPage] * H + g) * D;
    #pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            // channel 32 db + col: tokens 4 hg .. 4 hg + 3 and 8 + 4 hg .. 8 + 4 hg + 3
            const uint16_t* vrow = a.v_pages + (vt + 32 * db + col) * kPage;
            uint2 lo = *reinterpret_cast<const uint2*>(vrow + 4 * hg);
            uint2 hi = *reinterpret_cast<const uint2*>(vrow + 8 + 4 * hg);
            if (valid < kPage) {  // unwritten slots may hold NaN: zero them
              const int t0 = 4 * hg, t1 = 8 + 4 * hg;
              lo.x = t0 + 0 < valid ? (t0 + 1 < valid ? lo.x : lo.x & 0xFFFFu) : 0u;
              lo.y = t0 + 2 < valid ? (t0 + 3 < valid ? lo.y : lo.y & 0xFFFFu) : 0u;
              hi.x = t1 + 0 < valid ? (t1 + 1 < valid ? hi.x : hi.x & 0xFFFFu) : 0u;
              hi.y = t1 + 2 < valid ? (t1 + 3 < valid ? hi.y : hi.y & 0xFFFFu) : 0u;
            }
            const uint4 w4 = make_uint4(lo.x, lo.y, hi.x, hi.y);
            const bf16x8_t va = __builtin_bit_cast(bf16x8_t, w4);
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[c], o[db], 0, 0, 0);
          }
        }
      }
  }

  // ---- normalise and store: register r of block db holds channel
  // 32 db + 8 (r / 4) + 4 hg + r % 4 of query `col`
  const float lsum = sum_xor<32>(l);
  const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
  if (row_ok) {
    const int64_t orow = ((int64_t)(q0 + p) * a.num_q_heads + h) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = 32 * db + 8 * r4 + 4 * hg;
        const float x0 = o[db][4 * r4] * inv, x1 = o[db][4 * r4 + 1] * inv;
        const float x2 = o[db][4 * r4 + 2] * inv, x3 = o[db][4 * r4 + 3] * inv;
        if (a.out_f32)
          *reinterpret_cast<float4*>(static_cast<float*>(a.out) + orow + d0) =
              make_float4(x0, x1, x2, x3);
        else
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + orow + d0) =
              make_uint2(pack_bf16x2(x0, x1), pack_bf16x2(x2, x3));
      }
  }
}

}  // namespace pfb

void launch_prefill_bf16(const PrefillBf16Args& args, int head_dim, int64_t blocks,
                         hipStream_t st) {
  switch (head_dim) {
    case 64: pfb::prefill_bf16_kernel<64><<<(unsigned)blocks, pfb::kThreads, 0, st>>>(args); break;
    case 128: pfb::prefill_bf16_kernel<128><<<(unsigned)blocks, pfb::kThreads, 0, st>>>(args); break;
    case 256: pfb::prefill_bf16_kernel<256><<<(unsigned)blocks, pfb::kThreads, 0, st>>>(args); break;
  }
}

}  // namespace kvq
