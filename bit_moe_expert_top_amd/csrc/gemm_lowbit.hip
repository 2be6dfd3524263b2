// Expert FFN for prefill-sized groups: a grouped GEMM on the matrix cores with the low-bit
// codebook weights decoded into bf16 tiles in LDS.
//
// [Moet-README] release notes of -r23: the prefill MoE is FC1 + SwiGLU, then FC2, over the
// routed rows of each expert.  [Moet-QA]: 2-bit codes on {-4,-1,1,4}, a bf16 scale per 32
// along K.  [Strata-R9700] path 6: 3-bit codes on eight levels, an e4m3 scale / 64 per 64.
//
// Work item = (row tile of <= 128 grouped rows of one expert, column tile of the weight rows).
// A workgroup has WV waves (8; 4 for K of at most 512, two workgroups per CU); every wave
// computes all 128 rows x its own 32*NCT weight columns with v_mfma_f32_32x32x16_bf16 (4 x NCT
// MFMA tiles; 2 x NCT for an item of at most 64 rows).  The weights never pass through LDS: each lane
// loads and decodes straight into its MFMA B registers the 32-k field it supplies (lane l:
// weight row l % 32 of a column tile, k-half l / 32 of every 64-k step; for 2-bit codes that is
// exactly one scale group), with the format's own decode (lowbit_fmt.h).  Only the token rows
// (the A operand, shared by the workgroup's waves) are staged in LDS: direct global -> LDS loads into a
// four-deep ring, 16-byte chunks XOR-swizzled by row / 2 (conflict-free reads of 128-byte rows),
// one barrier per 64-k step; the packed codes and scales run in a four-slot register ring; codes
// are fetched two steps ahead, token rows three.  Per MFMA the LDS carries
// 0.5 KB of A reads (no B writes or reads), so the matrix cores rather than LDS bound the step.
// Work is handed out in blocks of 2 consecutive items x all column tiles, one block to the
// workgroups of one XCD at a time (workgroups are dispatched to the 8 XCDs round robin), so
// the weights of a column tile are shared through that XCD's L2 by the block's items (mostly
// of one expert: items are consecutive row chunks) and an item's token rows by its tiles.
// A workgroup's tasks run back to back through the same rings: when K is a multiple of 512 the
// last steps of a task already load the next task's first codes and token rows, so that task
// starts without a prologue (its loads overlap the end of the K loop and the epilogue).
// Token operand and decoded weights share the format's k-slot order: x comes permuted from the
// prepare kernel and FC1 writes h permuted, so A and B always agree.
//   FC1 column tile n (NCT = 2): wave w holds gate rows 32WVn + 32w + [0,32) and up rows
//       I + 32WVn + 32w + [0,32) as its two MFMA column tiles, so gate and up of one h column
//       sit in the same lane and register and SwiGLU is applied in the epilogue (h stored bf16).
//   FC2 column tile n: weight rows 32WV*NCT*n + 32*NCT*w + 32c + [0,32) (NCT = 2 when H is a
//       multiple of 512, else 1); the epilogue stores y (fp32).
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "lowbit_fmt.h"

namespace bitmoe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// D(32x32, f32) += A(32x16) * B(16x32).  Lane l supplies A row l%32 and B column l%32 for
// k = 8*(l/32) .. +7; it receives D[8*(j/4) + 4*(l/32) + j%4][l%32] in register j.
__device__ __forceinline__ f32x16 mfma_32x32x16_bf16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

constexpr int kBM = 128, kBK = 64;
constexpr int kAStage = kBM * kBK * 2;  // one step of token rows (bf16): 16 KB
// token rows run in a ring of 4 stages (as0..as3): stage = step % 4, a static index
constexpr int kGemmCUs = 256;           // workgroups per launch: 8 / WV per CU
typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt vmcnt(N) (gfx9 encoding; expcnt and lgkmcnt not waited on)
template <int N>
__device__ __forceinline__ void gemm_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | 0x70 | 0xF00 | ((N >> 4) << 14));
}

// One lane's 32-k field of one weight row for one step: the packed code words and the scale.
template <class F>
struct Field {
  uint32_t c[F::kFieldWords];
  uint32_t s;
};
// vector loads per field (the waits below count them)
template <class F>
constexpr int field_loads() { return F::kFieldWords == 3 ? 3 : 2; }

template <class F>
__device__ __forceinline__ void load_field(Field<F>& g, buf_rsrc rc, buf_rsrc rs, uint32_t co, uint32_t so) {
  const uint64_t c01 = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(rc, (int)co, 0, 0));
  g.c[0] = (uint32_t)c01;
  g.c[1] = (uint32_t)(c01 >> 32);
  if constexpr (F::kFieldWords == 3) g.c[2] = buf_load4(rc, co + 8u);
  if constexpr (F::kId == W2Fmt::kId)
    g.s = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, (int)so, 0, 0);
  else
    g.s = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rs, (int)so, 0, 0);
}

template <class F, int FC, int NCT, int WV>
__global__ __launch_bounds__(64 * WV, 8 / WV) void gemm_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, int rows_per_expert,
    int K, int width, int ktop, const uint16_t* __restrict__ asrc, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ plan, uint32_t asrc_bytes, void* __restrict__ out) {
  static_assert(FC == 2 || NCT == 2, "FC1 pairs a gate and an up column tile per wave");
  static_assert(WV == 4 || WV == 8, "8 waves per workgroup, or 4 (two workgroups per CU)");
  constexpr int kU = 16 / WV;  // 8-row token loads per wave and step (128 rows over WV waves)
  // one __shared__ object per stage: the compiler tracks the direct-to-LDS loads per object, so a
  // read of one stage waits only for that stage's loads (one array would wait for all of them)
  __shared__ __align__(16) uint8_t as0[kAStage];
  __shared__ __align__(16) uint8_t as1[kAStage];
  __shared__ __align__(16) uint8_t as2[kAStage];
  __shared__ __align__(16) uint8_t as3[kAStage];
  auto stage_ptr = [&](auto T_) -> uint8_t* {
    constexpr int T = decltype(T_)::value;
    return T == 0 ? as0 : (T == 1 ? as1 : (T == 2 ? as2 : as3));
  };
  int lane = wave_lane();
  asm volatile("" : "+v"(lane));  // lane-derived offsets are recomputed per tile, not held
  const int w = threadIdx.x / kWave;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int i32 = lane & 31, hk = lane >> 5;
  const int n_items = plan[0];
  const int4* items = reinterpret_cast<const int4*>(plan + 4);
  const int n_ntiles = FC == 1 ? width / (32 * WV) : rows_per_expert / (32 * WV * NCT);
  const uint32_t cbr = F::code_bytes((uint32_t)K), sbr = F::scale_bytes((uint32_t)K);
  const int nk = K / kBK;  // a multiple of 4 (K is a multiple of 256)
  // XCD-aware order: item blocks b = x, x + 8, ... go to XCD x (blockIdx % 8, for a grid that
  // is a multiple of 8); within a block the work runs column tile by column tile, the items of
  // the block side by side
  constexpr int kIB = 2;  // items per block (2 measured faster than 4 and 8)
  const int xcd = blockIdx.x & 7, nb_x = gridDim.x >> 3, lb = blockIdx.x >> 3;
  const int n_blocks = (n_items + kIB - 1) / kIB;
  const int blocks_x = n_blocks > xcd ? (n_blocks - xcd + 7) >> 3 : 0;
  const int per_block = kIB * n_ntiles;
  const int total_x = blocks_x * per_block;

  // Task p of this XCD's list = (item, column tile); the last block may hold one item, and the
  // tasks of its missing item are skipped (uniform per workgroup).
  struct Task {
    int p, nt_i, e, r0, nrows;
  };
  auto item_of = [&](int p, int& nt_i) {
    const int bl = p / per_block, rem = p - bl * per_block;
    nt_i = rem / kIB;
    return (xcd + 8 * bl) * kIB + (rem - nt_i * kIB);
  };
  auto next_task = [&](int p) {  // this workgroup's first task at or after p, or total_x
    for (; p < total_x; p += nb_x) {
      int nt;
      if (item_of(p, nt) < n_items) break;
    }
    return p;
  };
  auto task_at = [&](int p) {
    Task t;
    t.p = p;
    const int4 itm = items[item_of(p, t.nt_i)];
    t.e = itm.x;
    t.r0 = itm.y;
    t.nrows = itm.z;
    return t;
  };

  // The operands of one task are loaded through these resources and offsets; near the end of a
  // task they are switched to the next one (below), whose first loads then overlap the end of
  // this task's K loop and its epilogue.
  buf_rsrc ra, rc, rs;
  uint32_t aoff[kU], coff[NCT], soff[NCT];
  // ---- token rows (A): wave w loads rows (128/WV)w + 8u + lane/8 (u < 16/WV), 16-byte chunk
  //      position lane % 8 <- source chunk (lane % 8) ^ ((row / 2) % 8).  FC1 gathers rows of x (all
  //      of x is addressable); FC2 reads h rows r0.. of the item (based at r0: h may reach 2 GiB)
  auto arow_of = [&](int u) { return (128 / WV) * w + 8 * u + (lane >> 3); };
  // the source row of this lane's two A rows of task t: FC1 issues the perm loads here (branch
  // free, rows past the item clamped into it), read by set_rows
  auto row_lookup = [&](const Task& t, uint32_t(&tok)[kU]) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int rr = min(arow_of(u), t.nrows - 1);
      tok[u] = FC == 1 ? (uint32_t)perm[t.r0 + rr] : (uint32_t)rr;
    }
  };
  constexpr bool kGroup = F::kId == W2Fmt::kId;
  if constexpr (FC == 1) ra = make_rsrc(asrc, asrc_bytes);  // all of x, for every task
  auto set_rows = [&](const Task& t, const uint32_t(&tok)[kU]) {
    if constexpr (FC == 2) ra = make_rsrc(asrc + (size_t)t.r0 * K, (uint32_t)t.nrows * K * 2u);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int ar = arow_of(u);
      const uint32_t rowx = FC == 1 ? tok[u] / (uint32_t)ktop : tok[u];
      const int pos = lane & 7, src = pos ^ ((ar >> 1) & 7);
      const uint32_t ka = (kGroup ? 128u : 32u) * (uint32_t)(src >> 2) + 8u * (uint32_t)(src & 3);
      aoff[u] = ar < t.nrows ? (rowx * (uint32_t)K + ka) * 2u : kOffNone;
    }
  };
  // ---- weights (B): column tile c of this lane is weight row wrow[c]; per step the lane
  //      supplies one 32-k field of it.  2-bit codes come in groups of 4 steps (256 k): the
  //      lane's k-half hk owns the contiguous k [128 hk, 128 hk + 128) of the group, 32 k per
  //      step, so its 32 code bytes and 4 scales are fetched once per group (two 16-byte loads
  //      and one 8-byte load; the two halves of a row ask for 64 contiguous bytes at once,
  //      rather than 16 bytes of a different line every step).  3-bit codes come per step, the
  //      half hk owning k [32 hk, 32 hk + 32) of the step.  The token rows follow the same map.
  auto set_weights = [&](const Task& t) {
    const size_t ebase = (size_t)t.e * rows_per_expert;
    rc = make_rsrc(codes + ebase * cbr, (uint32_t)rows_per_expert * cbr);
    rs = make_rsrc(scales + ebase * sbr, (uint32_t)rows_per_expert * sbr);
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      const int wrow = FC == 1 ? (c == 0 ? 32 * WV * t.nt_i + 32 * w + i32 : width + 32 * WV * t.nt_i + 32 * w + i32)
                               : 32 * WV * NCT * t.nt_i + 32 * NCT * w + 32 * c + i32;
      if constexpr (kGroup) {
        coff[c] = (uint32_t)wrow * cbr + F::code_bytes(128u * hk);
        soff[c] = (uint32_t)wrow * sbr + F::scale_bytes(128u * hk);
      } else {
        coff[c] = (uint32_t)wrow * cbr + F::code_bytes(32u * hk);
        soff[c] = (uint32_t)wrow * sbr;  // one scale byte per step, shared by both halves
      }
    }
  };
  const uint32_t cstep = F::code_bytes(kBK), sstep = F::scale_bytes(kBK);
  // 2-bit: one lane's group (32 code bytes, 4 bf16 scales), in a two-slot ring (group g in
  // slot g % 2); 3-bit: one lane's field per step, in a four-slot ring (step kb in slot kb % 4)
  struct Group {
    uint32_t c[8];
    uint32_t s[2];
  };
  Group gr[kGroup ? 2 : 1][NCT];
  Field<F> fr[kGroup ? 1 : 4][NCT];
  auto load_group = [&](Group* gp, int g) {
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      const uint32_t co = coff[c] + (uint32_t)g * (4u * cstep), so = soff[c] + (uint32_t)g * (4u * sstep);
      const u32x4 lo = buf_load16(rc, co), hi = buf_load16(rc, co + 16u);
      const uint64_t sc = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(rs, (int)so, 0, 0));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        gp[c].c[i] = lo[i];
        gp[c].c[4 + i] = hi[i];
      }
      gp[c].s[0] = (uint32_t)sc;
      gp[c].s[1] = (uint32_t)(sc >> 32);
    }
  };
  auto load_codes = [&](Field<F>* f, int kb) {
#pragma unroll
    for (int c = 0; c < NCT; ++c)
      load_field<F>(f[c], rc, rs, coff[c] + (uint32_t)kb * cstep, soff[c] + (uint32_t)kb * sstep);
  };
  constexpr int kGroupLoads = 3 * NCT;  // vector loads per group (2-bit)
  // first k of the token chunk a lane loads, per step: 2-bit  256 (kb / 4) + 32 (kb % 4),
  // 3-bit 64 kb; plus, per lane, (128 or 32) * half + 8 * (chunk % 4)
  auto kstep = [&](int kb) -> uint32_t {
    return kGroup ? 256u * (uint32_t)(kb >> 2) + 32u * (uint32_t)(kb & 3) : 64u * (uint32_t)kb;
  };
  // token rows of step kb into stage T
  auto dma_a = [&](auto T_, int kb) {
    uint8_t* st = stage_ptr(T_);
#pragma unroll
    for (int u = 0; u < kU; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_t*)(st + 1024 * (kU * wu + u)), 16,
                                               (int)(aoff[u] + 2u * kstep(kb)), 0, 0, 0);
  };

  // A task started from nothing: the first codes (they overlap the row lookups), then the token
  // rows of steps 0..2; then the wait for step 0 and a barrier.
  constexpr int kPrologueCodeLoads = kGroup ? kGroupLoads : 2 * NCT * field_loads<F>();
  auto prologue = [&](const Task& t) {
    uint32_t tok[kU];
    row_lookup(t, tok);
    set_weights(t);
    if constexpr (kGroup) {
      load_group(gr[0], 0);
    } else {
      load_codes(fr[0], 0);
      load_codes(fr[1], min(1, nk - 1));
    }
    if constexpr (FC == 1) gemm_wait_vmcnt<kPrologueCodeLoads>();  // the row lookups
    set_rows(t, tok);
    dma_a(std::integral_constant<int, 0>{}, 0);
    dma_a(std::integral_constant<int, 1>{}, min(1, nk - 1));
    dma_a(std::integral_constant<int, 2>{}, min(2, nk - 1));
    gemm_wait_vmcnt<2 * kU>();  // the first codes and the token rows of step 0 (steps 1, 2 may fly)
    asm volatile("s_barrier" ::: "memory");
  };

  // A operand of MFMA tile m at k sub-step kk: row 32m + i32, 16-byte chunk 4hk + kk of the
  // step (the lane's k-half), stored at chunk position (4hk + kk) ^ ((row / 2) % 8)
  uint32_t apos[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) apos[kk] = (uint32_t)(i32 * 128 + 16 * ((4 * hk + kk) ^ ((i32 >> 1) & 7)));

  const int p_first = next_task(lb);
  if (p_first >= total_x) return;  // uniform over the workgroup
  Task cur = task_at(p_first);
  prologue(cur);
  for (;;) {
    const int p_next = next_task(cur.p + nb_x);
    const bool has_next = p_next < total_x;
    const Task nxt = task_at(has_next ? p_next : cur.p);
    // With K a multiple of 512 (a whole number of 8-step passes) the next task starts on token
    // stage 0 and code slot 0, so this task's last steps load its first codes and token rows
    // (the hand-over); otherwise it starts from its prologue after this task's epilogue.
    const bool pipe = has_next && nk % 8 == 0;
    const int r0 = cur.r0, nrows = cur.nrows, nt_i = cur.nt_i;

    // The rest of the tile runs on MT MFMA row tiles of 32: all 4, or 2 when the item has at most
    // 64 rows (an expert's last item often does), which halves its matrix work; rows past nrows
    // are zero in LDS either way.  The choice is uniform per workgroup.
    auto tile = [&](auto MT_) {
      constexpr int MT = decltype(MT_)::value;
      // the lane's epilogue rows and columns are derived here, per tile (held across the K loop
      // they would take some 30 registers)
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int ti32 = ln & 31, thk = ln >> 5;
      f32x16 acc[MT][NCT];
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int c = 0; c < NCT; ++c)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[m][c][i] = 0.f;
      // A operands of two sub-steps (read one sub-step ahead; sub-step 0 of a step is read during
      // the last sub-step of the step before)
      u32x4 av[2][MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) av[0][m] = *reinterpret_cast<const u32x4*>(as0 + apos[0] + 4096 * m);

      // Step kb (S8 = kb % 8; token stage S = kb % 4; 2-bit group slot P = S8 / 4), four 16-k
      // sub-steps, each: A from LDS (read one sub-step ahead), B decoded from the field, 4 x NCT
      // MFMAs.  Before the last sub-step's MFMAs the step hands over to the next one:
      //   1. wait for this lane's token rows of step kb + 1 and, before a group's first step, its
      //      codes (vector loads complete in issue order: those issued in step kb may stay in
      //      flight), then a barrier: every wave's rows of step kb + 1 are in LDS and every wave is
      //      done with step kb - 1 (it is past sub-step 2 of step kb).  The barrier is a bare
      //      s_barrier (with a compiler memory clobber): a __syncthreads fence would also drain the
      //      loads of the next steps still in flight, which nothing reads before their own wait;
      //   2. issue the next codes (2-bit: at a group's first step the next group, into the other
      //      slot; 3-bit: step kb + 2 into slot (S + 2) % 4) and the token rows of step kb + 3
      //      into stage (S + 3) % 4, which held step kb - 1.  Past the end of the task these are
      //      the next task's first group / steps 0, 1 and its steps 0..2 (pipe), or the last
      //      group / step fetched again into those free places, so the load counts never change;
      //   3. read sub-step 0 of step kb + 1, so its LDS latency hides behind the MFMAs of the
      //      last sub-step of step kb (the waves leave the barrier together).
      const int ng = nk >> 2;
      auto step = [&](auto S8_, int kb) {
        constexpr int S8 = decltype(S8_)::value, S = S8 & 3, P = S8 >> 2;
        constexpr int kWait = kU + (kGroup && S == 1 ? kGroupLoads : 0);
        const uint8_t* st = stage_ptr(std::integral_constant<int, S>{});
        const uint8_t* sn = stage_ptr(std::integral_constant<int, (S + 1) & 3>{});
        const uint32_t* fw[NCT];
        typename F::Tab tab[NCT];
#pragma unroll
        for (int c = 0; c < NCT; ++c) {
          if constexpr (kGroup) {
            fw[c] = &gr[P][c].c[2 * S];
            tab[c] = F::table32((gr[P][c].s[S >> 1] >> (16 * (S & 1))) & 0xFFFFu);
          } else {
            fw[c] = fr[S][c].c;
            tab[c] = F::table32(fr[S][c].s);
          }
        }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          if (kk + 1 < 4) {
#pragma unroll
            for (int m = 0; m < MT; ++m)
              av[(kk + 1) & 1][m] = *reinterpret_cast<const u32x4*>(st + apos[kk + 1] + 4096 * m);
          } else {
            __builtin_amdgcn_sched_barrier(0);
            gemm_wait_vmcnt<kWait>();
            asm volatile("s_barrier" ::: "memory");
            if constexpr (kGroup) {
              if constexpr (S == 0) {
                const int g = (kb >> 2) + 1;
                load_group(gr[P ^ 1], g < ng ? g : (pipe ? 0 : ng - 1));
              }
            } else {
              const int f = kb + 2;
              load_codes(fr[(S + 2) & 3], f < nk ? f : (pipe ? f - nk : nk - 1));
            }
            const int an = kb + 3;
            dma_a(std::integral_constant<int, (S + 3) & 3>{}, an < nk ? an : (pipe ? an - nk : nk - 1));
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int m = 0; m < MT; ++m) av[0][m] = *reinterpret_cast<const u32x4*>(sn + apos[0] + 4096 * m);
          }
#pragma unroll
          for (int c = 0; c < NCT; ++c) {
            const u32x4 bv = F::decode32(fw[c], tab[c], kk);
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[m][c] = mfma_32x32x16_bf16(av[kk & 1][m], bv, acc[m][c]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      };
      // nk is a multiple of 4 (K of 256); two 2-bit groups per pass keep every slot index static.
      // In the last pass of a hand-over the resources switch to the next task between steps:
      // its row lookups and (2-bit) code offsets before step nk - 4, whose group load is its
      // first group; its token rows before step nk - 3, whose DMA is its step 0; (3-bit) its code
      // offsets before step nk - 2, whose field load is its step 0.
      int kb = 0;
      for (; kb + 8 <= nk; kb += 8) {
        const bool hand = pipe && kb + 8 == nk;
        uint32_t tok_n[kU] = {};
        step(std::integral_constant<int, 0>{}, kb);
        step(std::integral_constant<int, 1>{}, kb + 1);
        step(std::integral_constant<int, 2>{}, kb + 2);
        step(std::integral_constant<int, 3>{}, kb + 3);
        if (hand) {
          row_lookup(nxt, tok_n);
          if constexpr (kGroup) set_weights(nxt);
        }
        step(std::integral_constant<int, 4>{}, kb + 4);
        if (hand) set_rows(nxt, tok_n);
        step(std::integral_constant<int, 5>{}, kb + 5);
        if constexpr (!kGroup) {
          if (hand) set_weights(nxt);
        }
        step(std::integral_constant<int, 6>{}, kb + 6);
        step(std::integral_constant<int, 7>{}, kb + 7);
      }
      if (kb < nk) {  // nk % 8 == 4: no hand-over (pipe is false)
        step(std::integral_constant<int, 0>{}, kb);
        step(std::integral_constant<int, 1>{}, kb + 1);
        step(std::integral_constant<int, 2>{}, kb + 2);
        step(std::integral_constant<int, 3>{}, kb + 3);
      }

      // ---- epilogue: lane holds column i32 of each tile, rows 32m + 8(j/4) + 4hk + j%4.  The
      //      stores go through a buffer resource that spans the item's nrows rows, so the rows
      //      past the item are dropped by its bound (no test per value); the lane's row 4hk and
      //      column are in a base offset, the rest of the row is uniform.
      constexpr uint32_t kEl = FC == 1 ? 2u : 4u;  // bytes per element: h bf16, y fp32
      const buf_rsrc ro = make_rsrc(reinterpret_cast<uint8_t*>(out) + (size_t)r0 * width * kEl,
                                    (uint32_t)nrows * (uint32_t)width * kEl);
      const uint32_t col = FC == 1 ? (uint32_t)(32 * (WV * nt_i + w) + F::pos32(ti32))
                                   : (uint32_t)(32 * WV * NCT * nt_i + 32 * NCT * w + ti32);
      const uint32_t vo = ((uint32_t)(4 * thk) * (uint32_t)width + col) * kEl;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const uint32_t ro_off = vo + (uint32_t)(32 * m + 8 * (j >> 2) + (j & 3)) * (uint32_t)width * kEl;
          if constexpr (FC == 1) {
            const float gt = acc[m][0][j], up = acc[m][1][j];
            const float hv = gt * __builtin_amdgcn_rcpf(1.0f + __expf(-gt)) * up;  // silu(gate) * up
            __builtin_amdgcn_raw_buffer_store_b16((unsigned short)f32_to_bf16_rne(hv), ro, (int)ro_off, 0, 0);
          } else {
            // y is read once, by the combine: non-temporal stores (aux bit 1; FC2 -3 % at T=8192)
#pragma unroll
            for (int c = 0; c < NCT; ++c)
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[m][c][j]), ro, (int)(ro_off + 32u * c * kEl), 0,
                                                    2);
          }
        }
      }
    };
    if (2 * nrows <= kBM)
      tile(std::integral_constant<int, 2>{});
    else
      tile(std::integral_constant<int, 4>{});
    if (!has_next) break;
    cur = nxt;
    if (pipe) {
      // the next task's first codes and token rows of steps 0..2 are in flight (issued by the last
      // steps, before this epilogue's stores): wait for its codes of step 0 (3-bit: steps 0, 1
      // come one per step) and its rows of step 0, then a barrier.  Its step 0 refills the stage of
      // this task's last step only after the barrier of its own step 0.
      gemm_wait_vmcnt<kGroup ? 2 * kU : 2 * kU + NCT * field_loads<F>()>();
      asm volatile("s_barrier" ::: "memory");
    } else {
      // every wave is done reading the token stages before the prologue refills them: an
      // LDS-only wait and a bare barrier (a __syncthreads fence would also wait for this tile's
      // h / y stores, which nothing in this workgroup reads)
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt not waited on
      asm volatile("s_barrier" ::: "memory");
      prologue(cur);
    }
  }
  // the last task's loads past its end (copies of its last stage) land before the workgroup ends
  gemm_wait_vmcnt<0>();
}

// Short K (at most 8 steps of 64, e.g. FC2 of a layer with I = 512): two 4-wave workgroups per
// CU, whose barriers are independent, so one's task start and epilogue overlap the other's
// MFMAs (3-bit FC2 at I = 512: -13 %); longer K: one 8-wave workgroup per CU, which loads each
// item's token rows once for twice the columns (prefill FC1 and FC2 +5 % on 4 waves).
template <class F, int FC, int NCT, int WV>
static hipError_t launch_gemm_wv(const void* codes, const void* scales, int rows, int K, int width,
                                 int ktop, const uint16_t* asrc, const int32_t* perm,
                                 const int32_t* plan, uint32_t asrc_bytes, void* out, hipStream_t s) {
  gemm_kernel<F, FC, NCT, WV><<<kGemmCUs * 8 / WV, 64 * WV, 0, s>>>(
      (const uint8_t*)codes, (const uint8_t*)scales, rows, K, width, ktop, asrc, perm, plan, asrc_bytes, out);
  return hipGetLastError();
}
template <class F, int FC, int NCT>
static hipError_t launch_gemm(const void* codes, const void* scales, int rows, int K, int width,
                              int ktop, const uint16_t* asrc, const int32_t* perm,
                              const int32_t* plan, uint32_t asrc_bytes, void* out, hipStream_t s) {
  return K <= 8 * kBK ? launch_gemm_wv<F, FC, NCT, 4>(codes, scales, rows, K, width, ktop, asrc, perm, plan, asrc_bytes, out, s)
                      : launch_gemm_wv<F, FC, NCT, 8>(codes, scales, rows, K, width, ktop, asrc, perm, plan, asrc_bytes, out, s);
}

hipError_t launch_lowbit_gemm_fc1(const LowbitWeights& w, int H, int I, int k, const uint16_t* xp,
                                  const int32_t* perm, const int32_t* plan, int max_items, int T,
                                  uint16_t* hbuf, hipStream_t s) {
  (void)max_items;
  const uint32_t xb = (uint32_t)((size_t)T * H * 2);
  if (w.fmt == W2Fmt::kId)
    return launch_gemm<W2Fmt, 1, 2>(w.w1_codes, w.w1_scales, 2 * I, H, I, k, xp, perm, plan, xb, hbuf, s);
  if (w.fmt == W3Fmt::kId)
    return launch_gemm<W3Fmt, 1, 2>(w.w1_codes, w.w1_scales, 2 * I, H, I, k, xp, perm, plan, xb, hbuf, s);
  return hipErrorInvalidValue;
}

hipError_t launch_lowbit_gemm_fc2(const LowbitWeights& w, int H, int I, int k,
                                  const uint16_t* hbuf, const int32_t* plan, int max_items, int T,
                                  float* y, hipStream_t s) {
  (void)max_items;
  const uint32_t hb = (uint32_t)((size_t)T * k * I * 2);
  // 512 weight rows per column tile when H allows, else 256 (H is a multiple of 256)
  const bool wide = H % 512 == 0;
  if (w.fmt == W2Fmt::kId)
    return wide ? launch_gemm<W2Fmt, 2, 2>(w.w2_codes, w.w2_scales, H, I, H, 1, hbuf, nullptr, plan, hb, y, s)
                : launch_gemm<W2Fmt, 2, 1>(w.w2_codes, w.w2_scales, H, I, H, 1, hbuf, nullptr, plan, hb, y, s);
  if (w.fmt == W3Fmt::kId)
    return wide ? launch_gemm<W3Fmt, 2, 2>(w.w2_codes, w.w2_scales, H, I, H, 1, hbuf, nullptr, plan, hb, y, s)
                : launch_gemm<W3Fmt, 2, 1>(w.w2_codes, w.w2_scales, H, I, H, 1, hbuf, nullptr, plan, hb, y, s);
  return hipErrorInvalidValue;
}

// ------------------------------------------------------------------ debug decode
// One thread per (row, 32-k field): the field loader, table32 and decode32 of the grouped GEMM
// (operand op of a field holds its k-slots 8 op .. 8 op + 7), written in natural k order.
template <class F>
__global__ __launch_bounds__(256) void debug_dequant_gemm_kernel(const uint8_t* __restrict__ codes,
                                                                 const uint8_t* __restrict__ scales, int rows,
                                                                 int K, float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int fpr = K / 32;
  if (i >= (int64_t)rows * fpr) return;
  const int row = (int)(i / fpr), f = (int)(i - (int64_t)row * fpr);
  const uint32_t cbr = F::code_bytes((uint32_t)K), sbr = F::scale_bytes((uint32_t)K);
  const buf_rsrc rc = make_rsrc(codes, (uint32_t)rows * cbr);
  const buf_rsrc rs = make_rsrc(scales, (uint32_t)rows * sbr);
  Field<F> g;
  load_field<F>(g, rc, rs, (uint32_t)row * cbr + F::code_bytes(32u * f), (uint32_t)row * sbr + F::scale_bytes(32u * f));
  const typename F::Tab tab = F::table32(g.s);
  float* o = out + (int64_t)row * K + 32 * f;
#pragma unroll
  for (int op = 0; op < 4; ++op) {
    const u32x4 v = F::decode32(g.c, tab, op);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int slot = 8 * op + 2 * d;
      o[F::slot_k(slot)] = bf16_to_f32(v[d] & 0xFFFFu);
      o[F::slot_k(slot + 1)] = bf16_to_f32(v[d] >> 16);
    }
  }
}

hipError_t launch_debug_dequant_gemm(const LowbitWeights& w, int H, int I, int e, int which, float* out,
                                     hipStream_t s) {
  const int rows = which == 1 ? 2 * I : H;
  const int K = which == 1 ? H : I;
  const uint8_t* codes = (const uint8_t*)(which == 1 ? w.w1_codes : w.w2_codes);
  const uint8_t* scales = (const uint8_t*)(which == 1 ? w.w1_scales : w.w2_scales);
  const int64_t n = (int64_t)rows * (K / 32);
  const unsigned grid = (unsigned)((n + 255) / 256);
  if (w.fmt == W2Fmt::kId) {
    const size_t cb = (size_t)e * rows * W2Fmt::code_bytes(K), sb = (size_t)e * rows * W2Fmt::scale_bytes(K);
    debug_dequant_gemm_kernel<W2Fmt><<<grid, 256, 0, s>>>(codes + cb, scales + sb, rows, K, out);
  } else if (w.fmt == W3Fmt::kId) {
    const size_t cb = (size_t)e * rows * W3Fmt::code_bytes(K), sb = (size_t)e * rows * W3Fmt::scale_bytes(K);
    debug_dequant_gemm_kernel<W3Fmt><<<grid, 256, 0, s>>>(codes + cb, scales + sb, rows, K, out);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace bitmoe
