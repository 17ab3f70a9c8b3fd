// Token-wise linear layers on the packed [T, d] stream: C = A W^T with bf16 MFMA tiles.
//
// Hugging Face blog "Continuous batching from first principles", section "Attention":
// layer normalisation and matrix multiplications are token-wise, each token's output
// depends on that token only, so they run on the packed stream with no regard for how
// requests are concatenated. hassanahmed "How continuous batching speeds up LLM serving":
// selective batching batches exactly these shape-agnostic operations. zhangchitc
// "continuous-batching", section "Inside the kernel": the new keys and values go into the
// KV cache before attention reads it back; the QKV epilogue here writes them straight into
// their pages, so no separate append pass touches them again.
//
// Work-group = 128 rows (tokens) x 128 or 256 columns (features), 4 waves as 2 x 2, each
// wave 64 x 64 or 64 x 128 = tiles of v_mfma_f32_32x32x16_bf16. K steps go through LDS,
// double-buffered (one barrier per step; the next step's global loads overlap the current
// step's MFMAs). The product is formed transposed, C^T = W A^T, so that a lane owns one
// token and four consecutive features per accumulator group: row-major stores (C, Q, K
// pages) are 8-byte vectors, and the transposed V pages get one element per lane with
// consecutive lanes on consecutive positions.
#include <type_traits>

#include "cb_device.h"

namespace cb {

namespace {

constexpr int kGM = 128;                          // rows (tokens) per work-group
constexpr int kXcds = 8;                          // XCDs work-groups are dealt over (MI355X)

__device__ __forceinline__ f32x16 mfma_g(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// scheduler groups for __builtin_amdgcn_sched_group_barrier
constexpr int kGSchedMfma = 0x0008;
constexpr int kGSchedDsRead = 0x0100;

}  // namespace

// BN = columns (features) per work-group: 128 (K steps of 64) or 256 (K steps of 32, so the
// double-buffered tiles still fit two work-groups per CU). Each of the 4 waves owns a 64 x
// BN/2 block: 2 x BN/64 tiles of 32 x 32.
template <int BN, int EPI>
__global__ __launch_bounds__(256, 2) void gemm_bt_kernel(GemmArgs g) {
  constexpr int BK = BN == 256 ? 32 : 64;
  constexpr int GS = BK;                          // LDS row stride (elements), unpadded
  constexpr int TA = kGM * GS, TB = BN * GS;      // one stage of A / B in LDS
  constexpr int NA = kGM * BK / 8 / 256;          // 16-byte chunks per thread per stage
  constexpr int NB = BN * BK / 8 / 256;
  constexpr int CPR = BK / 8;                     // 16-byte chunks per row
  // Chunk c of row r sits at chunk slot c ^ ((r / RP) % CPR), RP = rows per 256 bytes. Then
  // the 16 lanes of a quarter-wave hit 16 different 16-byte bank groups both when they
  // store (RP rows x CPR chunks) and when they read one chunk of 16 consecutive rows.
  constexpr int RP = 16 / CPR;
  auto slot = [](int r, int c) { return r * GS + ((c ^ ((r / RP) % CPR)) * 8); };
  constexpr int TN = BN / 64;                     // 32-wide feature tiles per wave
  __shared__ __align__(16) uint16_t lds[2 * (TA + TB)];
  __shared__ int32_t slot_blk[kGM], slot_off[kGM];
  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
  const int col = lane & 31, grp = lane >> 5;
  const int wm = wave & 1, wn = wave >> 1;
  // Work-group b runs on XCD b % 8. When the column tiles split evenly over the XCDs, XCD x
  // takes column tiles [x*nt/8, (x+1)*nt/8) for every row tile, consecutive work-groups on
  // an XCD sharing one weight tile: each weight tile then comes from HBM into one XCD's L2
  // once, instead of into every XCD.
  int mt_i = blockIdx.x, nt_i = blockIdx.y;
  {
    const int mtiles = gridDim.x, ntiles = gridDim.y;
    if (ntiles % kXcds == 0) {
      const int b = blockIdx.y * mtiles + blockIdx.x;
      const int x = b % kXcds, k = b / kXcds;
      const int per = ntiles / kXcds;
      nt_i = x * per + k / mtiles;
      mt_i = k % mtiles;
    }
  }
  const int m0 = mt_i * kGM, n0 = nt_i * BN;
  const int nk = g.K / BK;
  const uint16_t* A = static_cast<const uint16_t*>(g.a);
  const uint16_t* B = static_cast<const uint16_t*>(g.b);

  if constexpr (EPI == 1) {        // the cache slot of each row this work-group writes
    if (tid < kGM) {
      int blk = -1, off = 0;
      const int t = m0 + tid;
      if (t < g.M) {
        const int r = find_request(g.cu_q_lens, g.num_reqs, t);
        const int p = g.ctx_lens[r] + (t - g.cu_q_lens[r]);
        blk = g.block_tables[static_cast<int64_t>(r) * g.max_blocks + p / kBlockSize];
        off = p % kBlockSize;
        if (static_cast<unsigned>(blk) >= static_cast<unsigned>(g.num_blocks)) {
          note_violation(true);
          blk = -1;
        }
      }
      slot_blk[tid] = blk;
      slot_off[tid] = off;
    }
  }

  // two register sets: tile t is requested at the start of step t-2 and stored to LDS at the
  // end of step t-1, so its global loads have two steps of MFMA work to hide behind
  u32x4 ra[2][NA], rb[2][NB];
  // Per-thread byte offsets inside a K step are fixed; only the uniform step offset moves,
  // so the loads go through buffer resources (base + range in scalar registers, the offset
  // in one vector register) and need no per-load address arithmetic. Rows past M read row
  // M-1 (their products are never stored), so no load is predicated; the resource ranges
  // cover exactly this work-group's rows of A and B.
  uint32_t offa[NA], offb[NB];
#pragma unroll
  for (int u = 0; u < NA; ++u) {
    const int c = tid + 256 * u, row = min(c / CPR, g.M - 1 - m0);
    offa[u] = static_cast<uint32_t>((row * g.K + (c % CPR) * 8) * 2);
  }
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    const int c = tid + 256 * u;
    offb[u] = static_cast<uint32_t>(((c / CPR) * g.K + (c % CPR) * 8) * 2);
  }
  const int rows_a = min(kGM, g.M - m0);
  const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(A + static_cast<int64_t>(m0) * g.K), 0, rows_a * g.K * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(B + static_cast<int64_t>(n0) * g.K), 0, BN * g.K * 2, kBufferFlags);
  auto load = [&](int ks, int set) {
    const int so = ks * BK * 2;
#pragma unroll
    for (int u = 0; u < NA; ++u) ra[set][u] = __builtin_amdgcn_raw_buffer_load_b128(rsa, offa[u], so, 0);
#pragma unroll
    for (int u = 0; u < NB; ++u) rb[set][u] = __builtin_amdgcn_raw_buffer_load_b128(rsb, offb[u], so, 0);
  };
  auto store = [&](int buf, int set) {
    uint16_t* la = lds + buf * (TA + TB);
    uint16_t* lb = la + TA;
#pragma unroll
    for (int u = 0; u < NA; ++u) {
      const int c = tid + 256 * u;
      *reinterpret_cast<u32x4*>(la + slot(c / CPR, c % CPR)) = ra[set][u];
    }
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int c = tid + 256 * u;
      *reinterpret_cast<u32x4*>(lb + slot(c / CPR, c % CPR)) = rb[set][u];
    }
  };

  // acc[tn][tm]: C^T tile of features wn*BN/2 + tn*32 .. and tokens wm*64 + tm*32 ..
  f32x16 acc[TN][2];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn)
#pragma unroll
    for (int tm = 0; tm < 2; ++tm)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[tn][tm][i] = 0.f;

  // FULL: the step issues its loads unconditionally (the steady state), so the compiler's wait
  // before each register set is stored counts exactly the loads issued after it; a load
  // issued on some paths only makes it wait, on every path, as if it were never issued,
  // draining the loads for two steps ahead before the store of the next tile.
  auto step = [&](int ks, int set, auto full) {  // set = ks % 2
    if (decltype(full)::value || ks + 2 < nk) load(ks + 2, set);
    __builtin_amdgcn_sched_barrier(0);           // the loads go out before the step's products
    const uint16_t* la = lds + set * (TA + TB);
    const uint16_t* lb = la + TA;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 fa[2], fb[TN];
#pragma unroll
      for (int t = 0; t < 2; ++t)
        fa[t] = *reinterpret_cast<const bf16x8*>(la + slot(wm * 64 + t * 32 + col, kk * 2 + grp));
#pragma unroll
      for (int t = 0; t < TN; ++t)
        fb[t] = *reinterpret_cast<const bf16x8*>(lb + slot(wn * (BN / 2) + t * 32 + col, kk * 2 + grp));
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int tm = 0; tm < 2; ++tm) acc[tn][tm] = mfma_g(fb[tn], fa[tm], acc[tn][tm]);
    }
    // operand reads run ahead of the MFMAs that use them
    __builtin_amdgcn_sched_group_barrier(kGSchedDsRead, 2 + TN, 0);
#pragma unroll
    for (int k = 0; k < (BK / 16 - 1) * 2 * TN; ++k) {
      __builtin_amdgcn_sched_group_barrier(kGSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kGSchedDsRead, 1, 0);
    }
    if (ks + 1 < nk) store(set ^ 1, set ^ 1);   // tile ks+1: LDS buffer and register set (ks+1)%2
    __syncthreads();
  };
  // (a K of one step also loads step 1, which its buffer resources read as zeros or as
  // bytes never used)
  load(0, 0);
  load(1, 1);
  store(0, 0);
  __syncthreads();
  int ks = 0;
  for (; ks + 3 < nk; ks += 2) {
    step(ks, 0, std::true_type{});
    step(ks + 1, 1, std::true_type{});
  }
  for (; ks < nk; ++ks) step(ks, ks & 1, std::false_type{});

  // epilogue: lane owns token m0 + wm*64 + tm*32 + col and, per group q4 of accumulator
  // elements, features n0 + wn*BN/2 + tn*32 + 8*q4 + 4*grp + (0..3)
  const int qd = g.num_q_heads * g.head_dim, kd = g.num_kv_heads * g.head_dim;
#pragma unroll
  for (int tm = 0; tm < 2; ++tm) {
    const int mrow = wm * 64 + tm * 32 + col;
    const int m = m0 + mrow;
    if (m >= g.M) continue;
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int n = n0 + wn * (BN / 2) + tn * 32 + q4 * 8 + grp * 4;
        const f32x16& av = acc[tn][tm];
        const u32x2 w = u32x2{pack_bf16x2(av[q4 * 4], av[q4 * 4 + 1]), pack_bf16x2(av[q4 * 4 + 2], av[q4 * 4 + 3])};
        if (EPI == 0 || n < qd) {
          const int ldc = EPI == 0 ? g.N : qd;
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(g.c) + static_cast<int64_t>(m) * ldc + n) = w;
        } else {
          const int blk = slot_blk[mrow];
          if (blk < 0) continue;
          const int off = slot_off[mrow];
          const bool is_k = n < qd + kd;
          const int nn = n - qd - (is_k ? 0 : kd);
          const int hh = nn / g.head_dim, d = nn % g.head_dim;
          const int64_t page = static_cast<int64_t>(blk) * g.num_kv_heads + hh;
          if (is_k) {
            *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(g.k_cache) +
                                      (page * kBlockSize + off) * g.head_dim + d) = w;
          } else {
            uint16_t* vp = static_cast<uint16_t*>(g.v_cache) + (page * g.head_dim + d) * kBlockSize + off;
#pragma unroll
            for (int j = 0; j < 4; ++j) vp[j * kBlockSize] = static_cast<uint16_t>(j & 1 ? w[j >> 1] >> 16 : w[j >> 1] & 0xffffu);
          }
        }
      }
  }
}

hipError_t launch_gemm(const GemmArgs& g, int epilogue, hipStream_t s) {
  if (g.M == 0) return hipSuccess;
  // 256-wide column tiles read each token tile once for twice the features; they are used
  // when they still make at least two work-groups per CU (and, for the QKV epilogue, when
  // no tile straddles the Q/K/V boundaries)
  const int64_t mt = (g.M + kGM - 1) / kGM;
  const bool sections_ok = epilogue == 0 || ((g.num_q_heads * g.head_dim) % 256 == 0 &&
                                             (g.num_kv_heads * g.head_dim) % 256 == 0);
  const bool wide = g.N % 256 == 0 && g.K % 32 == 0 && sections_ok && mt * (g.N / 256) >= 2 * kNumCUs;
  if (wide) {
    const dim3 grid(static_cast<unsigned>(mt), g.N / 256);
    if (epilogue == 1)
      hipLaunchKernelGGL((gemm_bt_kernel<256, 1>), grid, dim3(256), 0, s, g);
    else
      hipLaunchKernelGGL((gemm_bt_kernel<256, 0>), grid, dim3(256), 0, s, g);
  } else {
    const dim3 grid(static_cast<unsigned>(mt), g.N / 128);
    if (epilogue == 1)
      hipLaunchKernelGGL((gemm_bt_kernel<128, 1>), grid, dim3(256), 0, s, g);
    else
      hipLaunchKernelGGL((gemm_bt_kernel<128, 0>), grid, dim3(256), 0, s, g);
  }
  return hipGetLastError();
}

CB_VIOLATION_READER(violations_gemm)

}  // namespace cb
