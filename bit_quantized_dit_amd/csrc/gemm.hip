// Dual-branch W4A4 GEMM on gfx950 ("W4A4 Quantization for Inference on
// Wan2.2-I2V-A14B (ICME 2026 Challenge)", sec. 3.3):
//
//   Y[t][n] = sum_p Q(X_J / s_J)[t][p] Q(s_J * W_J)[n][p]      (MXFP4 x MXFP4)
//           + sum_i X_O[t][i] W_O[n][i]                         (BF16 x BF16)
//
// Both branches accumulate into the same fp32 registers:
//   - the J branch with v_mfma_scale_f32_32x32x64_f8f6f4 in FP4 (E2M1) mode, whose
//     per-lane E8M0 scale operands apply 2^(c-127) per 32-element K block to each
//     operand, i.e. exactly the MXFP4 block scaling;
//   - the O branch with v_mfma_f32_32x32x16_bf16 (lane l feeds row l%32 and
//     values 8(l/32)..8(l/32)+7 of a 16-wide step).
// (The 32x32 shapes sustain close to the FP4 peak from a single wavefront per SIMD;
// the 16x16x128 shape issues at about half that rate.)
// Operand roles: src0 = weight rows (32 features), src1 = activation rows (32
// tokens).  Lane l of a 32x32x64 operand feeds row l%32 and the 32-code K chunk l/32
// (16 bytes, even K index in the low nibble) together with the E8M0 byte of that
// chunk; lane l of the result holds token l%32 and features 8q + 4(l/32) + r, r < 4,
// in registers 4q + r, stored as four float4.
//
// Operand layout: both code operands arrive in the tiled order (1 KiB per 16-row
// block and 128-code step, chunk-swizzled as in LDS), so every DMA instruction reads
// one contiguous KiB; the step-major scale words are one contiguous run per step.
//
// Tiling: a 512-thread workgroup (8 wavefronts, 2 token halves x 4 feature quarters,
// two per SIMD) owns a 256-token x 256-feature output tile; each wavefront a
// 128 x 64 sub-tile (4 x 2 MFMA tiles, 128 fp32 accumulator registers per lane), so
// that one wavefront's LDS waits and barrier waits are covered by the MFMAs of its
// SIMD partner.  The 256 x 256 tile (the largest whose fp32 accumulators fit the
// CU's registers) keeps the global traffic per MFMA at the level that the per-CU
// vector memory path sustains.  The K loop walks 128-code steps (64 bytes per row).
// Operands move HBM/L2 -> LDS with buffer_load ... lds (no VGPR staging) into a ring
// of STAGES slots; STAGES-1 steps are in flight while the MFMAs of the current step
// run.  Each slot holds 256 + 256 rows of 64 bytes plus one 32-bit word of four E8M0
// codes per row (read from the step-major scale arrays, so that one wavefront's 64
// words are one contiguous 256-byte request).  After the FP4 steps the same ring
// streams the outlier branch: 32 bf16 values of X_O and W_O per row are again 64
// bytes, so each BF16 step has the slot layout of an FP4 step (without scales) and
// feeds v_mfma_f32_32x32x16_bf16 into the same accumulators.
// 16-byte chunks are XOR-swizzled by row so that fragment reads are bank-conflict
// free (the DMA writes each wavefront's 1 KiB contiguously, so the swizzle lives in
// the tiled code layout, and in the source addresses of the bf16 gather).
// Buffer descriptors cover exactly the tile's valid rows: rows past the token or
// feature tail read as zero, with no masking in the loop.
//
// Tile order: workgroups are dispatched round-robin over the 8 XCDs, each with its
// own L2, and the persistent workgroup b runs tiles b, b + G, b + 2G, ... with G a
// multiple of 8, so all of its tiles map to one XCD.  The linear tile id is remapped
// so that each XCD owns a contiguous range of tiles, ordered in groups of GROUP_M
// token panels, so that the workgroups resident on one XCD share A (token) and B
// (feature) panels in its L2.
#include "w4a4_device.h"
#include "w4a4_internal.h"

#include <type_traits>

namespace w4a4 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int G_THREADS = 512;               // 8 wavefronts: 2 per SIMD
constexpr int BT = 256;                      // tokens per workgroup tile
constexpr int BF = 256;                      // features per workgroup tile (the tile grid's width)
constexpr int FF = 2;                        // 32-feature MFMA tiles per wavefront (64 features)
constexpr int ROW_BYTES = 64;                // 128 FP4 codes per row per K step
constexpr int A_OFF = 0;                     // slot layout: A codes | B codes | A scales | B scales
constexpr int B_OFF = BT * ROW_BYTES;
constexpr int AS_OFF = (BT + BF) * ROW_BYTES;
constexpr int BS_OFF = AS_OFF + BT * 4;
constexpr int SLOT_BYTES = BS_OFF + BF * 4;  // 34 KiB
constexpr int STAGES = 4;
constexpr int GROUP_M = 4;
constexpr int NUM_XCD = 8;

__device__ __forceinline__ int swz(int row, int chunk) {
    return row * ROW_BYTES + ((chunk ^ ((row >> 2) & 3)) << 4);
}

// Block id -> (token tile, feature tile): XCD-contiguous ranges, grouped order.
// 32-bit arithmetic: the launcher keeps the tile count below 2^31.
__device__ __forceinline__ void tile_of(uint32_t bid, uint32_t nt_m, uint32_t nt_n, uint32_t& tm, uint32_t& tn) {
    const uint32_t total = nt_m * nt_n;
    const uint32_t q = total / NUM_XCD, r = total % NUM_XCD;
    const uint32_t x = bid % NUM_XCD, j = bid / NUM_XCD;
    const uint32_t id = (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + j;
    const uint32_t per_group = GROUP_M * nt_n;
    const uint32_t g = id / per_group;
    const uint32_t first_m = g * GROUP_M;
    const uint32_t gsize = nt_m - first_m < (uint32_t)GROUP_M ? nt_m - first_m : (uint32_t)GROUP_M;
    const uint32_t in_g = id - g * per_group;
    tn = in_g / gsize;
    tm = first_m + (in_g - tn * gsize);
}

// Epilogue variants.  EPI_F32: out is fp32 Y [T][N].  EPI_GELU: out is bf16 H [T][N]
// with H = bf16(gelu_tanh(bf16(Y))) applied to each fp32 output in the epilogue (the
// FFN up projection feeding the down projection, sec. 3.1 / 3.5), bit-identical to the
// standalone GELU pass over this kernel's Y.  EPI_QUANT: H is not stored; the
// epilogue goes on to the down layer's activation prep of H (sec. 3.2 / 3.3) and
// writes its A_q, A_s and X_O (QuantDst), bit-identical to the act-prep pass over H.
constexpr int EPI_F32 = 0, EPI_GELU = 1, EPI_QUANT = 2;
//
// Split K for the last, partial round of tiles (the plan is gemm_split_plan): the
// tiles [0, full) run whole; each remaining tile runs as `split` work items over
// consecutive ranges of its K steps, each writing its fp32 accumulators to its own
// 256 KiB block of `part` in register order.  A second launch (REDUCE) gives each
// wavefront sub-tile of each remaining tile a one-wavefront workgroup, which sums that
// sub-tile's parts of the blocks in range order and runs the variant's epilogue on the
// sum (eight workgroups per tile, so the partial sums stream through many CUs).
struct SplitArgs {
    float* part;
    int64_t full;
    int32_t split;
};
// Launch modes: whole tiles only (every split quantity a compile-time constant, so the
// code is that of a kernel without the split), the split launch, the reduce launch,
// and half tiles: the tail tiles [full, ntiles) of the 256 x 256 grid each run as two
// 256-token x 128-feature items, with four wavefronts along the tokens (64 each) and
// two along the features, one B row block per wavefront, and four loads per step.
constexpr int MODE_WHOLE = 0, MODE_SPLIT = 1, MODE_REDUCE = 2, MODE_HALF = 3;
//
// Persistent: workgroup b walks the tiles b, b + G, b + 2G, ... of the grouped order
// (G = grid size, one workgroup per CU; b and b + G sit on the same XCD), and its ring
// of LDS slots runs on across tile boundaries: the last steps of one tile already
// fetch the first steps of the next, whose operands are then in flight while this
// tile's last MFMAs and its epilogue run.  The refill that the last step would issue
// waits until the epilogue, which restages the accumulators through that free slot.
template <int EPI, int MODE>
__global__ __launch_bounds__(G_THREADS, 1) void gemm_w4a4_kernel(
    const uint8_t* __restrict__ Aq, const uint8_t* __restrict__ As, const uint16_t* __restrict__ XO,
    int64_t T, const uint8_t* __restrict__ Bq, const uint8_t* __restrict__ Bs_rows,
    const uint16_t* __restrict__ WO, int64_t N, int64_t k_pad, int64_t k_ld, void* __restrict__ out,
    int vec_store, QuantDst qd, SplitArgs sp) {
    float* __restrict__ Y = reinterpret_cast<float*>(out);
    uint16_t* __restrict__ H = reinterpret_cast<uint16_t*>(out);
    // the ring, then 1 KiB per wavefront that only the null loads of a tile's last
    // step write (never read)
    // the reduce launch stages its epilogue through one slot and fetches nothing
    constexpr int SMEM_BYTES = MODE == MODE_REDUCE ? SLOT_BYTES : STAGES * SLOT_BYTES + (G_THREADS / 64) * 1024;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM_BYTES];

    // this instance's tile: BF features (the grid stays 256 wide: ::w4a4::BF), FT
    // 32-token MFMA tiles per wavefront, WT wavefronts along the tokens, NB B row blocks
    // of 16 rows per wavefront per step, DPS loads per wavefront per step
    constexpr int BF = MODE == MODE_HALF ? 128 : ::w4a4::BF;
    constexpr int FT = BF == 256 ? 4 : 2;   // 32-token MFMA tiles per wavefront
    constexpr int WT = BT / (FT * 32);
    constexpr int NB = BF / 128;
    constexpr int DPS = 2 + NB + 1;
    constexpr int AS_OFF = (BT + BF) * ROW_BYTES;
    constexpr int BS_OFF = AS_OFF + BT * 4;
    static_assert(BS_OFF + BF * 4 <= SLOT_BYTES && WT * (BF / 64) == G_THREADS / 64, "tile geometry");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave-uniform (SGPR); a reduce workgroup is one wavefront standing in for wavefront
    // blockIdx % 8 of its tile
    const int wave = MODE == MODE_REDUCE ? (int)(blockIdx.x & 7) : __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wt = wave % WT;    // which FT * 32 tokens of the tile
    const int wf = wave / WT;    // which 64 features of the tile
    const int l32 = lane & 31;
    const int lh = lane >> 5;    // which 32-code half of a 64-code MFMA step this lane feeds
    const int64_t nt_m = (T + BT - 1) / BT, nt_n = (N + ::w4a4::BF - 1) / ::w4a4::BF;
    const int64_t ntiles = nt_m * nt_n;
    // work items: the whole tiles [0, sp.full), then sp.split K ranges of each later
    // tile; the REDUCE launch has one item per wavefront sub-tile of each later tile
    const int64_t nitems = MODE == MODE_REDUCE  ? (ntiles - sp.full) * (G_THREADS / 64)
                           : MODE == MODE_SPLIT ? sp.full + (ntiles - sp.full) * sp.split
                           : MODE == MODE_HALF  ? (ntiles - sp.full) * 2
                                                : sp.full;
    int64_t id = blockIdx.x;
    if (id >= nitems) return;

    const int64_t o_ld = k_ld * 2;       // bytes per row of X_O / W_O
    const int nkb = (int)(k_pad / 128);  // FP4 steps (128 codes = 64 bytes per row)
    const int nbf = (int)(k_ld / 32);    // BF16 steps (32 values = 64 bytes per row)
    const int nsteps = nkb + nbf;

    // A work item: a tile and the range [s0, s0 + len) of its K steps (steps are
    // numbered FP4 first, then BF16).  Its ring steps ns are at least STAGES, so that the
    // prefetch never reaches past the next item; the extra steps read null descriptors
    // (zeros) and add nothing.  part: the partial-sum block of a K range, or -1.
    struct Tile {
        int64_t t0, f0, part;
        int s0, len, ns;
        bool valid;
    };
    auto tile_at = [&](int64_t i) __attribute__((always_inline)) {
        Tile t;
        t.valid = i < nitems;
        // 32-bit: the launcher keeps the item count below 2^31
        uint32_t tile = MODE == MODE_HALF ? (uint32_t)(sp.full + (i >> 1)) : (uint32_t)i;
        t.part = -1;
        t.s0 = 0;
        t.len = nsteps;
        if (MODE == MODE_SPLIT && i >= sp.full) {
            const uint32_t q = (uint32_t)(i - sp.full), ns32 = (uint32_t)sp.split;
            const uint32_t tq = q / ns32, c = q - tq * ns32;
            tile = (uint32_t)sp.full + tq;
            t.part = q;
            t.s0 = (int)(c * (uint32_t)nsteps / ns32);
            t.len = (int)((c + 1) * (uint32_t)nsteps / ns32) - t.s0;
        }
        t.ns = t.len > STAGES ? t.len : STAGES;
        uint32_t tm = 0, tn = 0;
        if (t.valid) tile_of(tile, (uint32_t)nt_m, (uint32_t)nt_n, tm, tn);
        t.t0 = (int64_t)tm * BT;
        t.f0 = (int64_t)tn * ::w4a4::BF + (MODE == MODE_HALF ? (i & 1) * BF : 0);
        return t;
    };
    auto rows_a_of = [&](const Tile& t) __attribute__((always_inline)) { return T - t.t0 < BT ? T - t.t0 : (int64_t)BT; };
    // (the second half of a ragged last column of tiles may lie past N: no rows)
    auto rows_b_of = [&](const Tile& t) __attribute__((always_inline)) {
        return N - t.f0 < BF ? (N > t.f0 ? N - t.f0 : (int64_t)0) : (int64_t)BF;
    };

    // FP4 codes in the tiled order (1 KiB per 16-row block and step, the LDS swizzle
    // already applied): a tile's 16 row blocks start blk bytes apart.  Step-major
    // scales: step st's words of a tile's rows start at (st * rows_total + row0) * 4;
    // the step offset goes into the descriptor base (not soffset, which the range check
    // does not cover), so every descriptor spans exactly the tile's valid rows and tail
    // rows read zero.
    const int64_t blk = (int64_t)nkb * 1024;
    const v4i srd0 = make_srd(Aq, 0u);
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
    // per-lane source offsets of this wavefront's two 1 KiB row blocks per operand:
    // block b covers rows 16b..16b+15 and lands at LDS b*1024 as it lies in memory
    // for the FP4 codes (lane -> 16 contiguous bytes); the row-major bf16 outlier
    // operands are gathered into the same order: lane -> row 16b + lane/4, physical
    // chunk lane%4, logical chunk = physical ^ ((row >> 2) & 3)
    // (A: blocks 2w, 2w+1; B: the same, or block w when a wavefront has one B block)
    int voff[2], voffo[2], vb[2], vbo[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int row = 16 * (wave * 2 + h) + (lane >> 2);
        const int chunk = ((lane & 3) ^ ((row >> 2) & 3)) << 4;
        voff[h] = (wave * 2 + h) * (int)blk + lane * 16;
        voffo[h] = row * (int)o_ld + chunk;
        const int bb = NB == 2 ? wave * 2 + h : wave;
        const int rowb = 16 * bb + (lane >> 2);
        vb[h] = bb * (int)blk + lane * 16;
        vbo[h] = rowb * (int)o_ld + (((lane & 3) ^ ((rowb >> 2) & 3)) << 4);
    }
    // waves 0-3 copy the A scale words of rows 64w.., waves 4-7 the B scale words (in a
    // half tile waves 6 and 7 have no B rows: their scale loads go to the spare KiB)
    const bool sc_b = wave >= 4;
    const bool sc_live = !sc_b || (wave & 3) * 64 < BF;
    const int vsc = (64 * (wave & 3) + lane) * 4;
    const uint8_t* const sc_tbl = sc_b ? Bs_rows : As;   // this wavefront's step-major scale array
    const int64_t sc_total = sc_b ? N : T;               // its rows per step

    // Step st of tile tl: FP4 codes + scales for st < nkb, the 64-byte column slice
    // (st - nkb) of X_O / W_O for BF16 steps, and a null descriptor past the tile's
    // steps or for no tile (zero range: the loads return zeros and touch no memory).
    // Every step issues exactly DPS loads per wavefront, so the outstanding
    // count, and with it every wait below, is the same on every step.
    struct Src {
        v4i a, b, sc;   // A and B operands, this wavefront's scale words
        int so, fp4;
    };
    // Word-by-word scalar selects (a select of whole descriptors is lowered to a
    // table in scratch memory).
    auto pick = [&](bool c1, v4i x, bool c2, v4i y) __attribute__((always_inline)) {
        v4i r;
#pragma unroll
        for (int w = 0; w < 4; ++w)
            r[w] = __builtin_amdgcn_readfirstlane(c1 ? x[w] : (c2 ? y[w] : srd0[w]));
        return r;
    };
    auto src_of = [&](const Tile& tl, int u) __attribute__((always_inline)) {   // u: the item's step
        Src r;
        const int st = tl.s0 + u;
        const bool in = tl.valid && u < tl.len;
        const bool fp4 = in && st < nkb, bf = in && !fp4;
        const int sts = fp4 ? st : 0;
        const int64_t ra = rows_a_of(tl), rb = rows_b_of(tl);
        r.fp4 = fp4;
        r.a = pick(fp4, make_srd(Aq + (tl.t0 / 16) * blk, (uint32_t)((ra + 15) / 16 * blk)),
                   bf, make_srd(XO + tl.t0 * k_ld, (uint32_t)(ra * o_ld)));
        r.b = pick(fp4, make_srd(Bq + (tl.f0 / 16) * blk, (uint32_t)((rb + 15) / 16 * blk)),
                   bf, make_srd(WO + tl.f0 * k_ld, (uint32_t)(rb * o_ld)));
        r.sc = pick(fp4, make_srd(sc_tbl + ((int64_t)sts * sc_total + (sc_b ? tl.f0 : tl.t0)) * 4,
                                  (uint32_t)((sc_b ? rb : ra) * 4)), false, srd0);
        r.so = fp4 ? st * 1024 : (bf ? (st - nkb) * 64 : 0);
        return r;
    };
    // The common case, an FP4 step of the current item, with the per-item parts
    // precomputed: only the scale descriptor's base and the code offset move per step
    // (rebuilding and selecting every descriptor each step would cost more scalar
    // instructions than the scalar unit issues in a step's MFMA time).  The item's
    // first step s0 is folded into the code descriptors (base + s0 KiB, range - s0 KiB:
    // a row block b still passes the range check exactly when b is a valid block, since
    // s0 < nkb and a lane offset within a block is below 1 KiB) and into the scale
    // base, so the step offsets are the item's own.
    struct Fast {
        v4i a, b;
        const uint8_t* sc;   // this wavefront's scale words of the item's first step
        uint32_t sc_bytes;
    };
    auto fast_of = [&](const Tile& tl) __attribute__((always_inline)) {
        Fast f;
        const int64_t ra = rows_a_of(tl), rb = rows_b_of(tl);
        const int64_t s0 = tl.s0 < nkb ? tl.s0 : nkb;   // items of BF16 steps only never use it
        f.a = make_srd(Aq + (tl.t0 / 16) * blk + s0 * 1024, (uint32_t)((ra + 15) / 16 * blk - s0 * 1024));
        f.b = make_srd(Bq + (tl.f0 / 16) * blk + s0 * 1024, (uint32_t)((rb + 15) / 16 * blk - s0 * 1024));
        f.sc = sc_tbl + (s0 * sc_total + (sc_b ? tl.f0 : tl.t0)) * 4;
        f.sc_bytes = (uint32_t)((sc_b ? rb : ra) * 4);
        return f;
    };
    auto fast_src = [&](const Fast& f, int st) __attribute__((always_inline)) {   // st: the item's step
        Src r;
        r.fp4 = 1;
        r.a = f.a;
        r.b = f.b;
        r.sc = make_srd(f.sc + (int64_t)st * sc_total * 4, f.sc_bytes);
        r.so = st * 1024;
        return r;
    };
    auto slot_of = [&](int g) __attribute__((always_inline)) {   // LDS address of ring slot g % STAGES
        return lds0 + (uint32_t)((g & (STAGES - 1)) * SLOT_BYTES);
    };
    // live = false sends the (null) load to this wavefront's scratch KiB instead
    const uint32_t spare = lds0 + STAGES * SLOT_BYTES + wave * 1024;
    auto dma_code = [&](const Src& r, uint32_t slot, int h, int which, bool live = true) __attribute__((always_inline)) {
        const int vo = which == 0 ? (r.fp4 ? voff[h] : voffo[h]) : (r.fp4 ? vb[h] : vbo[h]);
        const uint32_t dst = slot + (which == 0 ? A_OFF + (wave * 2 + h) * 1024
                                                : B_OFF + (NB == 2 ? wave * 2 + h : wave) * 1024);
        dma16(which == 0 ? r.a : r.b, live ? dst : spare, vo, r.so);
    };
    auto dma_scale = [&](const Src& r, uint32_t slot, bool live = true) __attribute__((always_inline)) {
        const uint32_t dst = slot + (sc_b ? BS_OFF : AS_OFF) + (wave & 3) * 256;
        dma4(r.sc, live && sc_live ? dst : spare, vsc, 0);
    };
    auto issue = [&](const Src& r, uint32_t slot) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < 2; ++h) dma_code(r, slot, h, 0);
#pragma unroll
        for (int h = 0; h < NB; ++h) dma_code(r, slot, h, 1);
        dma_scale(r, slot);
    };

    // fragments of one half-step (64 FP4 codes or 16 bf16 values per row): 2 weight
    // + 4 activation operands of 16 bytes, at chunk 2h + lane/32 of the 64-byte row
    struct Frags {
        v4i b[FF], a[FT];          // 16 bytes per operand (32 FP4 codes or 8 bf16)
    };
    struct Scales {
        uint32_t b[FF], a[FT];     // scale words of a step (shifted in place at first use)
    };
    // g is the ring index of the step (its slot is g % STAGES)
    auto load_b = [&](Frags& f, int g, int h, int i) __attribute__((always_inline)) {
        const uint8_t* slot = smem + (g & (STAGES - 1)) * SLOT_BYTES;
        const int r = wf * 64 + i * 32 + l32;
        const uint4 q = *reinterpret_cast<const uint4*>(slot + B_OFF + swz(r, 2 * h + lh));
        f.b[i] = v4i{(int)q.x, (int)q.y, (int)q.z, (int)q.w};
    };
    auto load_a = [&](Frags& f, int g, int h, int j) __attribute__((always_inline)) {
        const uint8_t* slot = smem + (g & (STAGES - 1)) * SLOT_BYTES;
        const int r = wt * (FT * 32) + j * 32 + l32;
        const uint4 q = *reinterpret_cast<const uint4*>(slot + A_OFF + swz(r, 2 * h + lh));
        f.a[j] = v4i{(int)q.x, (int)q.y, (int)q.z, (int)q.w};
    };
    auto load_scale = [&](Scales& c, int g, int o) __attribute__((always_inline)) {   // o-th of 6 words
        const uint8_t* slot = smem + (g & (STAGES - 1)) * SLOT_BYTES;
        if (o < FF) c.b[o] = reinterpret_cast<const uint32_t*>(slot + BS_OFF)[wf * 64 + o * 32 + l32];
        else c.a[o - FF] = reinterpret_cast<const uint32_t*>(slot + AS_OFF)[wt * (FT * 32) + (o - FF) * 32 + l32];
    };
    // A row's scale word holds the E8M0 bytes of its four 32-blocks of the step, and lane
    // l feeds block 2h + l/32 in half-step h.  Each word is shifted right by 8 * (l / 32)
    // in place just before its first MFMA of the step (the wait for its LDS read falls
    // there anyway); the block's byte is then byte 2h, which the MFMA selects by
    // immediate: one shift per word and step instead of one per word and half-step.
    const int lsh = 8 * lh;
    auto load_half = [&](Frags& f, int g, int h, int o) __attribute__((always_inline)) {   // o-th of 6 operand reads
        if (o < FF) load_b(f, g, h, o);
        else load_a(f, g, h, o - FF);
    };

    v16f acc[FF][FT];
    auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < FF; ++i)
#pragma unroll
            for (int j = 0; j < FT; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    };
    // one MFMA of a half-step; the scale operands' byte select 2h picks the lane's E8M0
    // byte of the pre-shifted scale words
    auto mma_fp4 = [&](const Frags& f, const Scales& c, int h, int i, int j) __attribute__((always_inline)) {
        const v8i b = v8i{f.b[i][0], f.b[i][1], f.b[i][2], f.b[i][3], 0, 0, 0, 0};
        const v8i a = v8i{f.a[j][0], f.a[j][1], f.a[j][2], f.a[j][3], 0, 0, 0, 0};
        if (h == 0)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, acc[i][j], 4, 4, 0, (int)c.b[i], 0,
                                                                          (int)c.a[j]);
        else
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, acc[i][j], 4, 4, 2, (int)c.b[i], 2,
                                                                          (int)c.a[j]);
    };
    auto mma_bf16 = [&](const Frags& f, int i, int j) __attribute__((always_inline)) {
        const v8bf wb = __builtin_bit_cast(v8bf, f.b[i]);
        const v8bf xa = __builtin_bit_cast(v8bf, f.a[j]);
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wb, xa, acc[i][j], 0, 0, 0);
    };

    // Epilogue of tile tl.  Lane l holds token l32 and features 8q + 4*lh + r of each
    // MFMA tile; the wavefront restages its 128 x 64 sub-tile 16 tokens at a time
    // through its own part of a free ring slot, so that every store instruction writes
    // 4 whole rows of 64 features (256 contiguous bytes each) instead of 32 rows x 32
    // bytes.
    constexpr int SROW = 64 + 4;   // staged row stride in floats (16 bytes of padding)
    static_assert((G_THREADS / 64) * 16 * SROW * 4 <= SLOT_BYTES, "staging fits one ring slot");
    // fp32 Y: one 32 x 32 MFMA tile per wavefront at a time, all lanes writing; rows of
    // 128 bytes with the 16-byte chunk c of row r at chunk position c ^ ((r / 2) % 8), so
    // that the writes (a row per lane) and the reads (eight lanes per row) of any 16
    // consecutive lanes fall in distinct banks; each store instruction then writes 8 rows
    // x 128 contiguous bytes, i.e. whole cache lines.
    auto epilogue_f32 = [&](const Tile& tl, int g) __attribute__((always_inline)) {
        float* stage = reinterpret_cast<float*>(smem + (g & (STAGES - 1)) * SLOT_BYTES) + wave * (32 * 32);
        const bool full = rows_a_of(tl) == BT && rows_b_of(tl) == BF && vec_store;
        const int rr = lane >> 3, cc = lane & 7;   // the reading lane's row (mod 8) and chunk
#pragma unroll
        for (int j = 0; j < FT; ++j) {
#pragma unroll
            for (int i = 0; i < FF; ++i) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *reinterpret_cast<v4f*>(stage + l32 * 32 + (((2 * q + lh) ^ ((l32 >> 1) & 7)) << 2)) =
                        v4f{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int r = rr + 8 * k;
                    const v4f v = *reinterpret_cast<const v4f*>(stage + r * 32 + ((cc ^ ((r >> 1) & 7)) << 2));
                    const int64_t t = tl.t0 + wt * (FT * 32) + j * 32 + r;
                    const int64_t n = tl.f0 + wf * 64 + i * 32 + cc * 4;
                    if (full) {
                        __builtin_nontemporal_store(v, reinterpret_cast<v4f*>(Y + t * N + n));
                    } else if (t < T) {
                        if (vec_store && n + 3 < N) {
                            __builtin_nontemporal_store(v, reinterpret_cast<v4f*>(Y + t * N + n));
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (n + e < N) Y[t * N + n + e] = v[e];
                        }
                    }
                }
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // read before the next tile overwrites it
            }
        }
    };
    static_assert((G_THREADS / 64) * 32 * 32 * 4 <= SLOT_BYTES, "fp32 staging fits one ring slot");
    auto epilogue = [&](const Tile& tl, int g) __attribute__((always_inline)) {
        if constexpr (EPI == EPI_F32) {
            epilogue_f32(tl, g);
            return;
        }
        float* stage = reinterpret_cast<float*>(smem + (g & (STAGES - 1)) * SLOT_BYTES) + wave * (16 * SROW);
        const bool full = rows_a_of(tl) == BT && rows_b_of(tl) == BF && vec_store;
#pragma unroll
        for (int j = 0; j < FT; ++j) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                if ((l32 >> 4) == hh) {
#pragma unroll
                    for (int i = 0; i < FF; ++i)
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            *reinterpret_cast<v4f*>(stage + (l32 & 15) * SROW + i * 32 + 8 * q + 4 * lh) =
                                v4f{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                    acc[i][j][4 * q + 3]};
                }
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int r = (lane >> 4) + 4 * k;
                    const v4f v = *reinterpret_cast<const v4f*>(stage + r * SROW + (lane & 15) * 4);
                    const int64_t t = tl.t0 + wt * (FT * 32) + j * 32 + hh * 16 + r;
                    const int64_t n = tl.f0 + wf * 64 + (lane & 15) * 4;
                    if constexpr (EPI == EPI_GELU) {
                        const uint32_t h01 = gelu_tanh_bf16x2(v[0], v[1]), h23 = gelu_tanh_bf16x2(v[2], v[3]);
                        if (full) {
                            *reinterpret_cast<uint2*>(H + t * N + n) = make_uint2(h01, h23);
                        } else if (t < T) {
                            if (vec_store && n + 3 < N) {
                                *reinterpret_cast<uint2*>(H + t * N + n) = make_uint2(h01, h23);
                            } else {
                                const uint16_t hv[4] = {(uint16_t)h01, (uint16_t)(h01 >> 16), (uint16_t)h23,
                                                        (uint16_t)(h23 >> 16)};
#pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    if (n + e < N) H[t * N + n + e] = hv[e];
                            }
                        }
                    } else {
                        if (full) {
                            __builtin_nontemporal_store(v, reinterpret_cast<v4f*>(Y + t * N + n));
                        } else if (t < T) {
                            if (vec_store && n + 3 < N) {
                                __builtin_nontemporal_store(v, reinterpret_cast<v4f*>(Y + t * N + n));
                            } else {
#pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    if (n + e < N) Y[t * N + n + e] = v[e];
                            }
                        }
                    }
                }
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // read before the next half overwrites it
            }
        }
    };

    // Epilogue that quantizes for the down layer.  Each 32-feature MFMA tile of one token
    // is one 32-block of the down layer's K (f0 and the wavefront's offsets are
    // multiples of 32): lane l and lane l ^ 32 hold its 16 + 16 values.  Per value
    // h = bf16(gelu_tanh(bf16(y))) (the pair function the GELU epilogue uses); for a J
    // position q = fl32(h / s) = fl32(h * RN64(1 / s)) as in act-prep, and positions
    // past k_j inside the block are zero; the block's E8M0 code comes from the maximum
    // |q| of both lanes (a NaN propagates and gives 0xFF with zero nibbles); each lane
    // converts its 16 values into 8 bytes and one exchange with lane ^ 32 (v_perm on the
    // received word) gives each lane 8 contiguous bytes of the block's 16, stored into
    // the tiled A_q; lane l < 32 stores the scale byte.  Outlier features (f >= k_j)
    // store h into X_O.
    // The tile's 256 reciprocals RN64(1 / s) (zero past k_j) are copied once into the
    // free ring slot g (every wavefront has finished reading it at the last step's
    // barrier; its refill waits until after the epilogue), and each lane reads its four
    // consecutive ones per group q from LDS when it needs them.
    auto epilogue_quant = [&](const Tile& tl, int g) __attribute__((always_inline)) {
        const int64_t kj = qd.k_j;
        const int64_t nkb_d = qd.k_pad / 128;
        const uint32_t sel_lo = lh ? 0x05040100u : 0x01000504u;
        const uint32_t sel_hi = lh ? 0x07060302u : 0x03020706u;
        double* const rs = reinterpret_cast<double*>(smem + (g & (STAGES - 1)) * SLOT_BYTES);
        if constexpr (MODE == MODE_REDUCE) {   // one wavefront: its own 64 features
            const int r = wf * 64 + lane;
            const int64_t f = tl.f0 + r;
            rs[r] = f < kj ? qd.rinv[f] : 0.0;
        } else if (tid < BF) {
            const int64_t f = tl.f0 + tid;
            rs[tid] = f < kj ? qd.rinv[f] : 0.0;
        }
        __syncthreads();
        // One 32-feature block (MFMA tile column i) for the wavefront's FT token tiles.
        // ALL_J: every feature of the block is a J position (the common case): no
        // masking, no X_O stores, and GELU without its NaN canonicalization, since a NaN
        // of any payload encodes the same (scale 0xFF, zero nibbles).
        auto quant_block = [&](auto all_j_c, int i) __attribute__((always_inline)) {
            constexpr bool ALL_J = decltype(all_j_c)::value;
            const int64_t fb = tl.f0 + wf * 64 + i * 32;   // the block's first feature (wave-uniform)
            // the lane's features are fb + o, o = 4 lh + 8q + e in [0, 32); the J
            // positions among them are o < jl
            const int64_t jlo = kj - fb;
            const bool has_j = ALL_J || jlo > 0;
            const int jl = ALL_J ? 32 : (jlo > 0 ? (jlo >= 32 ? 32 : (int)jlo) : 0);
            const double* const rl = rs + (wf * 64 + i * 32 + 4 * lh);   // the lane's first feature in the tile
#pragma unroll
            for (int j = 0; j < FT; ++j) {
                const int64_t t = tl.t0 + wt * (FT * 32) + j * 32 + l32;
                const bool tok = t < T;
                uint32_t hw[8];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if constexpr (ALL_J) {
                        hw[2 * q] = gelu_tanh_bf16x2_raw(acc[i][j][4 * q], acc[i][j][4 * q + 1]);
                        hw[2 * q + 1] = gelu_tanh_bf16x2_raw(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
                    } else {
                        hw[2 * q] = gelu_tanh_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]);
                        hw[2 * q + 1] = gelu_tanh_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
                    }
                }
                if (has_j) {
                    float qv[16];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const double4 rq = *reinterpret_cast<const double4*>(rl + 8 * q);
                        const double rr[4] = {rq.x, rq.y, rq.z, rq.w};
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int r = 4 * q + e;
                            const uint32_t w = hw[r / 2];
                            const float x = __uint_as_float((r & 1) ? (w & 0xFFFF0000u) : (w << 16));
                            qv[r] = (float)((double)x * rr[e]);
                            if constexpr (!ALL_J) qv[r] = 4 * lh + 8 * q + e < jl ? qv[r] : 0.0f;
                        }
                    }
                    float m4[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        m4[q] = __builtin_elementwise_maximum(
                            __builtin_elementwise_maximum(__builtin_fabsf(qv[4 * q]), __builtin_fabsf(qv[4 * q + 1])),
                            __builtin_elementwise_maximum(__builtin_fabsf(qv[4 * q + 2]), __builtin_fabsf(qv[4 * q + 3])));
                    uint32_t mb = __float_as_uint(__builtin_elementwise_maximum(
                        __builtin_elementwise_maximum(m4[0], m4[1]), __builtin_elementwise_maximum(m4[2], m4[3])));
                    const uint32_t pb = (uint32_t)__shfl_xor((int)mb, 32);
                    mb = pb > mb ? pb : mb;
                    const uint32_t code = e8m0_from_absbits(mb);
                    const float scale = __uint_as_float(__builtin_elementwise_max(code << 23, 0x00400000u));
                    uint32_t p0 = 0, p1 = 0;
                    p0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p0, qv[0], qv[1], scale, 0);
                    p0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p0, qv[2], qv[3], scale, 1);
                    p0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p0, qv[4], qv[5], scale, 2);
                    p0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p0, qv[6], qv[7], scale, 3);
                    p1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p1, qv[8], qv[9], scale, 0);
                    p1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p1, qv[10], qv[11], scale, 1);
                    p1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p1, qv[12], qv[13], scale, 2);
                    p1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p1, qv[14], qv[15], scale, 3);
                    // a NaN/Inf block: zero nibbles
                    p0 = code == 0xFFu ? 0u : p0;
                    p1 = code == 0xFFu ? 0u : p1;
                    // lane < 32 holds bytes {0,1,4,5} / {8,9,12,13} of the block, lane >= 32
                    // bytes {2,3,6,7} / {10,11,14,15}; after the exchange lane < 32 writes
                    // bytes 0..7 and lane >= 32 bytes 8..15
                    const uint32_t own = lh ? p1 : p0;
                    const uint32_t recv = (uint32_t)__shfl_xor((int)(lh ? p0 : p1), 32);
                    const uint32_t lo = __builtin_amdgcn_perm(own, recv, sel_lo);
                    const uint32_t hi = __builtin_amdgcn_perm(own, recv, sel_hi);
                    if (tok) {
                        const int r16 = (int)(t & 15);
                        uint8_t* dst = qd.aq + (((t >> 4) * nkb_d + (fb >> 7)) << 10) + (r16 << 6) +
                                       (((((int)(fb >> 5)) & 3) ^ (r16 >> 2)) << 4) + lh * 8;
                        *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
                        if (lh == 0) qd.as[(((fb >> 7) * T + t) << 2) + ((fb >> 5) & 3)] = (uint8_t)code;
                    }
                }
                if constexpr (!ALL_J) {
                    if (tok) {
                        // value r is feature fb + o, o = 4 lh + 8 (r / 4) + r % 4 in [0, 32); the
                        // outlier slots are the o in [kj - fb, N - fb)
                        const int64_t nhi = N - fb;
                        const int o_min = jl, o_max = nhi > 32 ? 32 : (int)nhi;
                        uint16_t* const xrow = qd.xo + t * qd.k_ld - jlo;
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int o = 4 * lh + 8 * (r / 4) + (r % 4);
                            if (o >= o_min && o < o_max)
                                xrow[o] = (uint16_t)((r & 1) ? (hw[r / 2] >> 16) : hw[r / 2]);
                        }
                    }
                }
            }
        };
#pragma unroll
        for (int i = 0; i < FF; ++i) {
            const int64_t fb = tl.f0 + wf * 64 + i * 32;
            if (fb >= N) continue;
            if (kj - fb >= 32) quant_block(std::true_type{}, i);
            else quant_block(std::false_type{}, i);
        }
    };

    // A K range's accumulators, in register order: each store writes 1 KiB, 16 bytes
    // per lane.  The REDUCE launch reads them back in the same order.
    auto part_ptr = [&](int64_t blk_idx) __attribute__((always_inline)) {
        return sp.part + blk_idx * (BT * BF) + wave * (FF * FT * 16 * 64) + lane * 4;
    };
    auto store_part = [&](const Tile& tl) __attribute__((always_inline)) {
        float* p = part_ptr(tl.part);
#pragma unroll
        for (int i = 0; i < FF; ++i)
#pragma unroll
            for (int j = 0; j < FT; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *reinterpret_cast<v4f*>(p + ((i * FT + j) * 4 + q) * 256) =
                        v4f{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
    };

    if constexpr (MODE == MODE_REDUCE) {
        // one wavefront's sub-tile of a later tile per workgroup (one wavefront): the sum
        // of its K ranges' blocks, first to last, then that wavefront's part of the
        // epilogue, staged through slot 0 (the epilogues are per wavefront)
        const int64_t q = id / (G_THREADS / 64);
        Tile tl;
        uint32_t tm = 0, tn = 0;
        tile_of((uint32_t)(sp.full + q), (uint32_t)nt_m, (uint32_t)nt_n, tm, tn);
        tl.t0 = (int64_t)tm * BT;
        tl.f0 = (int64_t)tn * BF;
        tl.part = -1;
        tl.s0 = 0;
        tl.len = tl.ns = 0;
        tl.valid = true;
        for (int c = 0; c < sp.split; ++c) {
            const float* p = part_ptr(q * sp.split + c);
#pragma unroll
            for (int i = 0; i < FF; ++i)
#pragma unroll
                for (int j = 0; j < FT; ++j)
#pragma unroll
                    for (int qq = 0; qq < 4; ++qq) {
                        const v4f v = *reinterpret_cast<const v4f*>(p + ((i * FT + j) * 4 + qq) * 256);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            acc[i][j][4 * qq + e] = c == 0 ? v[e] : acc[i][j][4 * qq + e] + v[e];
                    }
        }
        if constexpr (EPI == EPI_QUANT) epilogue_quant(tl, 0);
        else epilogue(tl, 0);
        return;
    }

    // Pipeline.  MFMAs issue in order, so the LDS fragment reads and the DMA issue
    // are interleaved one by one between the MFMAs of the other half-step, where
    // they co-execute with the matrix pipe (sched_barrier pins the order):
    //   half 0 of step st: 16 MFMAs on f0, interleaved with the 8 fragment reads of
    //                      half 1 (f1);
    //   sync:              wait for step st+1's DMA and for this wavefront's reads
    //                      of slot st, then one barrier (slot st is free, slot st+1
    //                      visible);
    //   half 1 of step st: 16 MFMAs on f1, interleaved with the 8 reads of half 0
    //                      of step st+1 (f0) and the 10 DMAs refilling slot st with
    //                      step st+STAGES.
    // At the sync point steps st+1..st+STAGES-1 are in flight; waiting for all but
    // the last STAGES-2 of them (vmcnt 10) leaves step st+1 landed.  Loads complete in
    // issue order among themselves, so a wait for at most n outstanding operations
    // leaves every load landed that has at least n loads issued after it.  Across a
    // tile boundary more is issued after the next tile's steps 1 and 2 (the null
    // loads of the last step, the epilogue's stores, the deferred refill), which only
    // makes those two waits stricter.  The FP4 steps run first, then the BF16 steps
    // of the outlier branch on the same ring.
    static_assert(STAGES == 4 && (DPS == 5 || DPS == 4), "vmcnt immediates below assume 4 x 5 or 4 x 4");
    Tile cur = tile_at(id);
#pragma unroll
    for (int st = 0; st < STAGES; ++st) issue(src_of(cur, st), slot_of(st));
    if constexpr (DPS == 5) asm volatile("s_waitcnt vmcnt(15)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
    __syncthreads();
    Frags f0, f1;
    Scales c0, c1;                 // scale words of the current and of the next step
    // half 0 fragments and scale words of a tile's first step (ring index g)
    auto load_first = [&](int g) __attribute__((always_inline)) {
#pragma unroll
        for (int o = 0; o < FF + FT; ++o) {
            load_half(f0, g, 0, o);
            load_scale(c0, g, o);
        }
    };
    load_first(0);
    zero_acc();

    constexpr int NM = FF * FT;   // MFMAs per half-step
    int base = 0;                 // ring index of the current item's step 0
    for (;;) {
        const int64_t next_id = id + gridDim.x;
        const Tile nxt = tile_at(next_id);
        const Fast fc = fast_of(cur);
        const int ns = cur.ns;
        // the item's FP4 steps come first: [0, nfp4) of its own steps
        const int nfp4 = cur.s0 >= nkb ? 0 : (nkb - cur.s0 < cur.len ? nkb - cur.s0 : cur.len);
        auto sync = [&]() __attribute__((always_inline)) {
            if constexpr (DPS == 5) asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
            else asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // slot st fully read
            __syncthreads();
        };
        // half 1 of step st; its DMA fetches ring step st + STAGES: this tile's, the
        // next tile's first steps, or at the last step nothing: null loads into the
        // spare KiB keep the load count of every step the same, and the refill of this
        // slot waits until the epilogue has staged through it
        auto refill = [&](int st) __attribute__((always_inline)) {
            const int s4 = st + STAGES;
            const bool here = s4 < ns;
            Tile tl = here ? cur : nxt;
            tl.valid = tl.valid && st + 1 < ns;
            return src_of(tl, here ? s4 : s4 - ns);
        };
        auto half1 = [&](int st, bool fp4, const Scales& cs, Scales& nx, const Src& r, bool dma)
            __attribute__((always_inline)) {
            const uint32_t slot = slot_of(base + st);
#pragma unroll
            for (int s = 0; s < NM; ++s) {
                if (fp4) mma_fp4(f1, cs, 1, s % FF, s / FF);
                else mma_bf16(f1, s % FF, s / FF);
                if (s < FF + FT) {
                    load_half(f0, base + st + 1, 0, s);
                    load_scale(nx, base + st + 1, s);
                }
                // the step's loads spread over the MFMAs: A blocks, B blocks, scales
                constexpr int D0 = NM >= 6 ? 1 : 0;
                if (s == D0 || s == D0 + 1) dma_code(r, slot, s - D0, 0, dma);
                if (s >= D0 + 2 && s < D0 + 2 + NB) dma_code(r, slot, s - D0 - 2, 1, dma);
                if (s == D0 + 2 + NB) dma_scale(r, slot, dma);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        // FP4 steps, unrolled by two so that the scale words of the current and the
        // next step alternate between c0 and c1 without a copy (a copy would wait for
        // every outstanding LDS read at the end of each step)
        auto fp4_step = [&](int st, Scales& cs, Scales& nx, bool fast) __attribute__((always_inline)) {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < NM; ++s) {
                if (s < FF) cs.b[s] >>= lsh;
                if (s % FF == 0) cs.a[s / FF] >>= lsh;
                mma_fp4(f0, cs, 0, s % FF, s / FF);
                if (s < FF + FT) load_half(f1, base + st, 1, s);
                __builtin_amdgcn_sched_barrier(0);
            }
            sync();
            __builtin_amdgcn_sched_barrier(0);
            if (fast) half1(st, true, cs, nx, fast_src(fc, st + STAGES), true);
            else half1(st, true, cs, nx, refill(st), st + 1 < ns);
        };
        // BF16 steps (and the null steps that pad short K); the scale words they load
        // are unused here
        auto bf16_step = [&](int st) __attribute__((always_inline)) {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < NM; ++s) {
                mma_bf16(f0, s % FF, s / FF);
                if (s < FF + FT) load_half(f1, base + st, 1, s);
                __builtin_amdgcn_sched_barrier(0);
            }
            sync();
            __builtin_amdgcn_sched_barrier(0);
            half1(st, false, c1, c0, refill(st), st + 1 < ns);
        };
        int st = 0;
        // steps whose refill is this item's FP4 step st + STAGES
        for (; st + 1 + STAGES < nfp4; st += 2) {
            fp4_step(st, c0, c1, true);
            fp4_step(st + 1, c1, c0, true);
        }
        for (; st + 1 < nfp4; st += 2) {
            fp4_step(st, c0, c1, false);
            fp4_step(st + 1, c1, c0, false);
        }
        if (st < nfp4) fp4_step(st++, c0, c1, false);
        for (; st < ns; ++st) bf16_step(st);

        // The last step's half 1 has already read the next tile's first fragments; they
        // are read again below so that no register holds them across the epilogue.
        if (MODE == MODE_SPLIT && cur.part >= 0) store_part(cur);
        else if constexpr (EPI == EPI_QUANT) epilogue_quant(cur, base + ns - 1);
        else epilogue(cur, base + ns - 1);
        if (!nxt.valid) break;
        __syncthreads();   // every wavefront is done with the staging slot
        issue(src_of(nxt, STAGES - 1), slot_of(base + ns - 1));
        base += ns;
        cur = nxt;
        id = next_id;
        load_first(base);
        zero_acc();
    }
}

// One persistent workgroup per CU (the LDS ring admits one), at most one per tile,
// and a multiple of the XCD count, so that a workgroup's tiles stay on its XCD.
static int64_t gemm_grid(int64_t tiles) {
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (cus[dev] == 0) {
        int c = 0;
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) c = 256;
        cus[dev] = c;
    }
    const int64_t g = cus[dev] >= NUM_XCD ? cus[dev] / NUM_XCD * NUM_XCD : cus[dev];
    return tiles < g ? tiles : g;
}

// Split plan: the tiles that fill whole rounds of SPLIT_SLOTS workgroups (the CU count
// of the part) run whole, and the remaining tail tiles (all tiles, when there are fewer
// than SPLIT_SLOTS) are each cut into `split` K ranges, so that the last round keeps
// most CUs busy.  A layer whose tiles are not split and all fit twice into the slots
// (at most 128 tiles) runs as half tiles (256 x 128): one round of half the length,
// with no partial sums.  (Half tiles for the tail after whole rounds were measured
// slower: the second launch's gap and the half tile's larger DMA share per FLOP
// outweigh the shorter last round: 57600 x 5120 -> 13824, 2297-2299 against 2282-2285
// us.)  A split is used only at 3 or more ranges per tile (at 2 the extra
// partial-sum traffic and the reduce launch eat most of what the shorter round saves),
// with at least SPLIT_MIN_STEPS K steps per range (a range pays about as much as a
// dozen steps for its partial-sum store, its pipeline fill and its share of the reduce
// launch).  Host logic only: the workspace size queries and the launch compute the same
// plan.
constexpr int64_t SPLIT_SLOTS = 256, SPLIT_MAX = 16, SPLIT_MIN = 3, SPLIT_MIN_STEPS = 16;

GemmSplit gemm_split_plan(int64_t T, int64_t N, int64_t k_pad, int64_t k_ld) {
    GemmSplit p;
    const int64_t tiles = T > 0 && N > 0 ? ((T + BT - 1) / BT) * ((N + BF - 1) / BF) : 0;
    p.full = tiles;
    p.split = 1;
    p.part_bytes = 0;
    p.half = 0;
    const int64_t tail = tiles < SPLIT_SLOTS ? tiles : tiles % SPLIT_SLOTS;
    if (tail == 0) return p;
    int64_t s = SPLIT_SLOTS / tail;
    if (s > SPLIT_MAX) s = SPLIT_MAX;
    const int64_t nsteps = k_pad / 128 + k_ld / 32;
    if (s > nsteps / SPLIT_MIN_STEPS) s = nsteps / SPLIT_MIN_STEPS;
    if (s < SPLIT_MIN) {
        if (2 * tail <= SPLIT_SLOTS && tail == tiles) {
            p.full = tiles - tail;
            p.half = 1;
        }
        return p;
    }
    p.full = tiles - tail;
    p.split = (int32_t)s;
    p.part_bytes = (size_t)(tail * s) * BT * BF * sizeof(float);
    return p;
}

namespace {

template <int EPI>
hipError_t launch_epi(const uint8_t* Aq, const uint8_t* As, const uint16_t* XO, int64_t T, const w4a4_packed& d,
                      void* out, int vec_store, const QuantDst& q, float* part, hipStream_t st) {
    const int64_t tiles = ((T + BT - 1) / BT) * ((d.d_out + BF - 1) / BF);
    const GemmSplit plan = gemm_split_plan(T, d.d_out, d.k_pad, d.k_ld);
    if (plan.split > 1 && !part) return hipErrorInvalidValue;
    const SplitArgs sp{part, plan.full, plan.split};
    if (plan.split == 1) {
        if (plan.full > 0)
            gemm_w4a4_kernel<EPI, MODE_WHOLE><<<dim3((unsigned)gemm_grid(plan.full)), G_THREADS, 0, st>>>(
                Aq, As, XO, T, d.B_q_tiles, d.B_s_rows, d.W_O, d.d_out, d.k_pad, d.k_ld, out, vec_store, q, sp);
        if (plan.half) {
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            gemm_w4a4_kernel<EPI, MODE_HALF><<<dim3((unsigned)gemm_grid(2 * (tiles - plan.full))), G_THREADS, 0, st>>>(
                Aq, As, XO, T, d.B_q_tiles, d.B_s_rows, d.W_O, d.d_out, d.k_pad, d.k_ld, out, vec_store, q, sp);
        }
        return hipGetLastError();
    }
    const int64_t items = plan.full + (tiles - plan.full) * plan.split;
    gemm_w4a4_kernel<EPI, MODE_SPLIT><<<dim3((unsigned)gemm_grid(items)), G_THREADS, 0, st>>>(
        Aq, As, XO, T, d.B_q_tiles, d.B_s_rows, d.W_O, d.d_out, d.k_pad, d.k_ld, out, vec_store, q, sp);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    gemm_w4a4_kernel<EPI, MODE_REDUCE><<<dim3((unsigned)((tiles - plan.full) * (G_THREADS / 64))), 64, 0, st>>>(
        Aq, As, XO, T, d.B_q_tiles, d.B_s_rows, d.W_O, d.d_out, d.k_pad, d.k_ld, out, vec_store, q, sp);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const uint8_t* Aq, const uint8_t* As, const uint16_t* XO, int64_t T,
                       const w4a4_packed& d, void* out, bool gelu_bf16, float* part, hipStream_t st) {
    if (T <= 0 || d.d_out <= 0) return hipSuccess;
    const int64_t tiles = ((T + BT - 1) / BT) * ((d.d_out + BF - 1) / BF);
    if (tiles > 0x7FFFFFFF / SPLIT_MAX) return hipErrorInvalidValue;
    // 32-bit buffer offsets: one tile's rows of codes must span < 2 GiB
    if ((int64_t)BT * (d.k_pad / 2) >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    // vector stores: 16 bytes (fp32) or 8 bytes (bf16) per lane, aligned when every row is
    const int vec_store = (d.d_out % 4 == 0) && (((uintptr_t)out & 15u) == 0);
    const QuantDst none{};
    if (gelu_bf16) return launch_epi<EPI_GELU>(Aq, As, XO, T, d, out, vec_store, none, part, st);
    return launch_epi<EPI_F32>(Aq, As, XO, T, d, out, vec_store, none, part, st);
}

hipError_t launch_gemm_quant(const uint8_t* Aq, const uint8_t* As, const uint16_t* XO, int64_t T,
                             const w4a4_packed& up, const QuantDst& q, float* part, hipStream_t st) {
    if (T <= 0 || up.d_out <= 0) return hipSuccess;
    const int64_t tiles = ((T + BT - 1) / BT) * ((up.d_out + BF - 1) / BF);
    if (tiles > 0x7FFFFFFF / SPLIT_MAX) return hipErrorInvalidValue;
    if ((int64_t)BT * (up.k_pad / 2) >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    // the epilogue's 32-blocks are the down layer's: its K is the up layer's N, and its
    // k_j + k columns are the up layer's outputs
    if (q.k_j + q.k != up.d_out || q.k_pad % 128 != 0 || q.k_pad < q.k_j) return hipErrorInvalidValue;
    return launch_epi<EPI_QUANT>(Aq, As, XO, T, up, nullptr, 0, q, part, st);
}

// rinv[p] = RN64(1 / s[J[p]]) for p < k_j (the reciprocal act-prep uses); zero codes
// and scale bytes for the 32-blocks from ceil(k_j / 32) to k_pad / 32 of every token
// (the fused epilogue writes the blocks that hold J positions); zero X_O columns
// k .. k_ld-1 of every token.
__global__ __launch_bounds__(256) void ffn_prologue_kernel(const float* __restrict__ s, const int32_t* __restrict__ J,
                                                           int64_t T, QuantDst q) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (int64_t p = g; p < q.k_j; p += stride) const_cast<double*>(q.rinv)[p] = 1.0 / (double)s[J[p]];
    const int64_t b0 = (q.k_j + 31) / 32, nb = q.k_pad / 32 - b0;   // pad blocks per token
    const int64_t nkb = q.k_pad / 128;
    for (int64_t e = g; e < T * nb; e += stride) {
        const int64_t t = e / nb, b = b0 + e % nb;
        const int r16 = (int)(t & 15);
        uint8_t* dst = q.aq + (((t >> 4) * nkb + (b >> 2)) << 10) + (r16 << 6) + ((((int)b & 3) ^ (r16 >> 2)) << 4);
        *reinterpret_cast<uint4*>(dst) = make_uint4(0u, 0u, 0u, 0u);
        q.as[(((b >> 2) * T + t) << 2) + (b & 3)] = 0;
    }
    const int64_t tail = q.k_ld - q.k;
    for (int64_t e = g; e < T * tail; e += stride) q.xo[(e / tail) * q.k_ld + q.k + e % tail] = 0;
}

hipError_t launch_ffn_prologue(const w4a4_packed& down, int64_t T, const QuantDst& q, hipStream_t st) {
    const int64_t work = q.k_j > T * (q.k_pad / 32) ? q.k_j : T * (q.k_pad / 32);
    if (work <= 0) return hipSuccess;
    int64_t blocks = (work + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    ffn_prologue_kernel<<<(unsigned)blocks, 256, 0, st>>>(down.s, down.J, T, q);
    return hipGetLastError();
}

}  // namespace w4a4
