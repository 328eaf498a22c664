// zi_kernels.hip -- gfx950 kernels of the tiled linear operator.
//
// One MFMA GEMM template covers the three products of a weight tile
// (memory-centric tiling of Y = XW, ZeRO-Infinity transformer-math page,
// section "Memory-centric tiling: operators bigger than the device"):
//   forward   Y_i  = X W_i          both operands reduction-contiguous
//   dX       dX   += dY_i W_i^T     the tile operand is read across its rows
//   dW       dW_i  = X^T dY_i       both operands are read across their rows
// The output C[p][q] is row-major with q contiguous.  The MFMA "A" operand is
// the one indexed by q (called Q), the "B" operand the one indexed by p
// (called P), so each lane's four consecutive accumulator registers land on
// four consecutive q, and every epilogue store is one 8- or 16-byte vector.
//
// Workgroup: 256 threads = 4 wave64s in a 2 x 2 arrangement over a
// 256 (p) x 256 (q) macro-tile; each wave owns 128 x 128 = 8 x 8 MFMA blocks
// of 16 x 16 (v_mfma_f32_16x16x32_{f16,bf16}, fp32 accumulators: 256 per lane,
// so the kernel runs one wave per SIMD).
//
// Memory pipeline.  With one wave per SIMD nothing hides a wait except work
// already queued, so global reads must be issued far ahead of their use.  Every
// operand is copied global -> LDS by the buffer unit (buffer_load ... lds,
// 16 bytes per lane), which needs no registers.  A step covers BK = 64
// reduction elements; one operand of one step (32 KiB) is a "unit", and the
// LDS holds a ring of five units (160 KiB).  While step s is multiplied (from
// registers), the fragments of step s + 1 are read from its two units and
// the next units are in flight: step s + 2's pair and the first unit of step
// s + 3.  Each wave waits only for the units it needs next (s_waitcnt
// vmcnt(N) with N = the copies still allowed in flight), meets the others at
// one barrier per step, and reads MFMA fragments from LDS:
//   * reduction-contiguous operand: rows of 64 reduction values (128 B, eight
//     16-byte chunks), so eight lanes fetch one whole 128-byte line of global
//     memory; chunk c of row r sits at c ^ ((r >> 1) & 7); a fragment is one
//     ds_read_b128 per lane;
//   * reduction-strided operand: kept in its natural layout, rows of 256
//     elements (512 B, sixteen 32-byte segments) per reduction index k;
//     segment s of row k sits at s ^ ((k & 3) | ((k >> 1) & 4)); a fragment
//     is two ds_read_b64_tr_b16 per lane.  That instruction, per 16 lanes, hands lane
//     j the (j % 4)-th element read by lanes 4e + j / 4 (e = 0..3); pointing
//     those 16 lanes at 4 consecutive rows x 4 four-element column groups gives
//     each lane 4 consecutive reduction values of one column: the MFMA layout.
// The LDS serves 256 bytes per clock (64 banks of 4 bytes): both layouts let
// every 16 lanes of a 16-byte read, and every 32 lanes of an 8-byte transposing
// read, fall on distinct banks.  Full 128-byte rows matter: the vector L1
// sends one request per 64-byte half line otherwise, and the number of
// requests it keeps in flight, not the L2's bandwidth, bounds the fill rate.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "zi_internal.h"

namespace zi {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int BK = kGemmStep;                        // reduction elements per step

// Epilogues: RNE to 16 bits; fp32; GeLU (A and H = GeLU(A) in 16 bits);
// accumulate into fp32 C; GeLU with A kept in fp32 (H still from the 16-bit A).
enum Epi { EPI_LP = 0, EPI_F32 = 1, EPI_GELU = 2, EPI_ACC = 3, EPI_GELU_F32A = 4 };

__device__ __forceinline__ uint32_t lds_addr(const char *p) { return (uint32_t)(uintptr_t)p; }

// ---- global -> LDS copies -------------------------------------------------------
//
// Reads go through raw buffer descriptors.  A lane whose element lies outside
// the operand gets the offset kOOB, past the descriptor's range; the buffer
// unit returns zeros for it, so ragged edges need no branches.

constexpr uint32_t kNumRecords = 0x40000000u;  // bytes covered by a descriptor
constexpr uint32_t kOOB = 0x40000000u;         // lane offset outside that range
constexpr uint32_t kRsrcWord3 = 0x00020000u;   // raw 32-bit buffer, gfx9 layout

typedef uint32_t rsrc_t __attribute__((ext_vector_type(4)));

// Buffer descriptor: 48-bit base, stride 0, kNumRecords bytes.  The base is
// the same for every lane; readfirstlane states so, keeping the descriptor in
// scalar registers where the instruction needs it.
__device__ __forceinline__ rsrc_t make_rsrc(const char *base, uint32_t records = kNumRecords) {
    const uint64_t b = (uint64_t)(uintptr_t)base;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
    return rsrc_t{lo, hi & 0xffffu, records, kRsrcWord3};
}

// rs with its base moved on by `bytes` (bases stay below 2^48, so the carry
// never reaches the stride field).
__device__ __forceinline__ rsrc_t rsrc_add(rsrc_t rs, uint64_t bytes) {
    const uint64_t b = (((uint64_t)rs[1] << 32) | rs[0]) + bytes;
    rs[0] = (uint32_t)b;
    rs[1] = (uint32_t)(b >> 32);
    return rs;
}

// One 16-byte-per-lane copy global -> LDS at lds_block + 16 * lane.  Written as
// inline assembly so that the compiler's wait-count pass, which cannot tell
// LDS stages apart, does not drain every copy in flight before each LDS read;
// completion is awaited explicitly (wait_and_barrier) before a stage is read.
//
// m0 is reserved to the compiler, which warns that it may not honour the
// clobber; the build's assembly check makes sure that no compiler-generated
// instruction touches m0 at all, so the warning is silenced here.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void copy16(rsrc_t rs, uint32_t lds_block, uint32_t voff) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_block);
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds"
        :
        : "s"(m0), "v"(voff), "s"(rs)
        : "memory", "m0");
}
#pragma clang diagnostic pop

// An operand unit holds one step (BK reduction values) of ROWS rows of an
// operand: ROWS * BK * 2 bytes, filled by NCOPY = ROWS / 32 copies per wave.
// Copy j of wave w fills bytes [(NCOPY w + j) * 1 KiB, +1 KiB) of the unit;
// lane l writes the 16 bytes at offset 16 l of that block.  Each wave reads
// the fragments of its half of the rows (WROWS = ROWS / 2: the workgroup's
// four waves form 2 x 2 over the macro-tile).

// Reduction-contiguous operand, element (r, k) at M[r * ld + k].  LDS rows of
// 64 reduction values (128 B, eight 16-byte chunks); chunk c of row r sits at
// c ^ ((r >> 1) & 7).  Eight lanes fetch one 128-byte row of global memory.
template <int ROWS>
struct RcOperand {
    static constexpr int NCOPY = ROWS / 32;
    static constexpr int WROWS = ROWS / 2;
    static constexpr int UNIT = ROWS * BK * 2;
    static_assert(ROWS % 64 == 0 && WROWS % 16 == 0, "rows come in 16-row fragments per wave");
    const char *base;  // &M[r0 * ld]
    uint32_t voff[NCOPY];

    __device__ __forceinline__ static int chunk_pos(int r, int c) { return c ^ ((r >> 1) & 7); }
    __device__ __forceinline__ static int chunk_of(int j, int wave, int lane) {
        const int pos = (wave * NCOPY + j) * 1024 + lane * 16;
        return chunk_pos(pos >> 7, (pos >> 4) & 7);
    }

    __device__ __forceinline__ void init(const uint16_t *M, int64_t ld, int64_t r0, int64_t rext,
                                         int wave, int lane) {
        base = reinterpret_cast<const char *>(M + r0 * ld);
#pragma unroll
        for (int j = 0; j < NCOPY; ++j) {
            const int r = ((wave * NCOPY + j) * 1024 + lane * 16) >> 7;
            voff[j] = (r0 + r < rext) ? (uint32_t)((r * ld + chunk_of(j, wave, lane) * 8) * 2) : kOOB;
        }
    }

    // Copy cursor: the descriptor of the next step of this operand to copy
    // (based at that step's first reduction index) and that index.  The
    // steps are copied in order, so the cursor only moves on.
    rsrc_t cur;
    int32_t ck;
    __device__ __forceinline__ void init_cursor() {
        cur = make_rsrc(base);
        ck = 0;
    }
    // The next step's descriptor and first reduction index k0; moves the
    // cursor on.  With an aligned reduction length a step lies wholly in range
    // or (past the last one) wholly out, which the record count expresses.
    template <bool ALIGNED, bool SPLIT>
    __device__ __forceinline__ rsrc_t take(int32_t red, int32_t &k0) {
        rsrc_t rs = cur;
        if constexpr (ALIGNED) rs[2] = ck < red ? kNumRecords : 0u;
        k0 = ck;
        cur = rsrc_add(cur, 2 * BK);
        ck += BK;
        return rs;
    }
    // Copy j of this wave of a step taken as (rs, k0) into the unit whose
    // part for this wave starts at LDS address `at`; in a ragged step, chunks
    // at or past the reduction length read as zero.
    template <bool ALIGNED>
    __device__ __forceinline__ void issue(const rsrc_t &rs, int32_t k0, int32_t red, uint32_t at, int wave,
                                          int lane, int j) const {
        uint32_t off = voff[j];
        if constexpr (!ALIGNED) off = k0 + chunk_of(j, wave, lane) * 8 < red ? off : kOOB;
        copy16(rs, at + j * 1024, off);
    }

    // Fragment reads (v_mfma_f32_16x16x32).  Fragment f of half ks (0, 1) of
    // a step holds rows wh * WROWS + 16 f + (lane & 15) and reduction values
    // 32 ks + 8 (lane >> 4) .. +7: one 16-byte read.  Its address is the
    // unit's, plus a per-lane part that depends on ks only through the
    // swizzle (flo[ks], fixed for the kernel), plus 16 f rows (a constant).
    uint32_t flo[2];
    __device__ __forceinline__ void init_reads(int wh, int lane) {
        const int r = lane & 15;  // the swizzle sees r modulo 16 (WROWS and 16 f are multiples of 16)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            flo[ks] = (uint32_t)((wh * WROWS + r) * 128 + (chunk_pos(r, ks * 4 + (lane >> 4)) << 4));
    }
    // Per-lane base of the reads of half ks in the unit at LDS address
    // `unit`: one add, hidden from the optimiser so that the constant parts of
    // the addresses stay in the instructions' offset fields.
    struct Bases { uint32_t b; };
    __device__ __forceinline__ Bases bases(uint32_t unit, int ks) const {
        Bases r{unit + flo[ks]};
        asm volatile("" : "+v"(r.b));
        return r;
    }
    __device__ __forceinline__ void frag(const Bases &b, int ks, int f, u32x4 &out) const {
        (void)ks;
        out = *reinterpret_cast<const __attribute__((address_space(3))) u32x4 *>((uintptr_t)(b.b + f * 16 * 128));
    }
};

// Reduction-strided operand, element (r, k) at M[k * ld + r].  LDS rows of
// ROWS elements (ROWB bytes, 32-byte segments) per reduction index k.  The
// segments of row k are permuted so that the eight rows one transposing read
// touches (k = 8 h + 4 t + 0..3 for two h) fall on eight different 32-byte
// bank groups: with rows of a multiple of 256 bytes, segment s of row k sits
// at s ^ ((k & 3) | ((k >> 1) & 4)); with rows of 128 bytes past such a
// multiple (row k then starts half a bank period after row k - 1, which sets
// bit 2 of the bank group from k's parity), at s ^ (((k >> 1) & 1) | ((k >> 2) & 2)).
// Both permute within aligned groups of 8 (of 4) segments, so within a row.
template <int ROWS>
struct RsOperand {
    static constexpr int NCOPY = ROWS / 32;
    static constexpr int WROWS = ROWS / 2;
    static constexpr int ROWB = ROWS * 2;
    static constexpr int UNIT = ROWB * BK;
    static_assert(ROWB % 256 == 0 || ROWB % 256 == 128, "row layouts of the swizzles above");
    static_assert(WROWS % 16 == 0, "rows come in 16-row fragments per wave");
    const char *base;   // &M[r0]
    const char *base2;  // &M2[r0]: reduction rows from `split` on (split = 0: none)
    int32_t split;
    int64_t ldb;        // ld in bytes
    uint32_t voff[NCOPY];

    __device__ __forceinline__ void set_split(const void *M2, int64_t split_, int64_t r0) {
        split = M2 ? (int32_t)split_ : 0;
        base2 = M2 ? reinterpret_cast<const char *>(static_cast<const uint16_t *>(M2) + r0) : base;
    }

    __device__ __forceinline__ static int seg_pos(int k, int s) {
        if constexpr (ROWB % 256 == 0)
            return s ^ ((k & 3) | ((k >> 1) & 4));
        else
            return s ^ (((k >> 1) & 1) | ((k >> 2) & 2));
    }

    __device__ __forceinline__ void init(const uint16_t *M, int64_t ld, int64_t r0, int64_t rext,
                                         int wave, int lane) {
        base = reinterpret_cast<const char *>(M + r0);
        base2 = base;
        split = 0;
        ldb = ld * 2;
#pragma unroll
        for (int j = 0; j < NCOPY; ++j) {
            const int pos = (wave * NCOPY + j) * 1024 + lane * 16;
            const int k = pos / ROWB;                        // LDS row
            const int s = seg_pos(k, (pos % ROWB) >> 5);     // logical 32-byte segment
            const int r = s * 16 + ((pos >> 4) & 1) * 8;     // first of 8 elements
            voff[j] = (r0 + r < rext) ? (uint32_t)(k * ldb + r * 2) : kOOB;  // rext % 8 == 0
        }
    }

    // Copy cursor: the descriptor of the next step of this operand to copy
    // (based at that step's first reduction row) and that row's index.  The
    // steps are copied in order, so the cursor only moves on: by BK rows, or
    // to M2's first row when it reaches `split` (a step never straddles it).
    rsrc_t cur, cur2;  // cur2: based at M2's first row
    int32_t ck;
    __device__ __forceinline__ void init_cursor() {
        cur = make_rsrc(base);
        cur2 = make_rsrc(base2);
        ck = 0;
    }
    // The next step's descriptor and first reduction index k0; moves the
    // cursor on (with selects, not a branch: the main loop stays one block).
    // Rows at or past the reduction length read as zero: row k of
    // the unit lies in bytes [k ldb, (k + 1) ldb) from the step's base, so a
    // record count that ends after the last valid row cuts the rest off.
    template <bool ALIGNED, bool SPLIT>
    __device__ __forceinline__ rsrc_t take(int32_t red, int32_t &k0) {
        rsrc_t rs = cur;
        const int32_t rem = red - ck;  // valid rows from ck on (none past the end)
        if constexpr (ALIGNED)
            rs[2] = rem > 0 ? kNumRecords : 0u;
        else
            rs[2] = rem <= 0 ? 0u : (rem >= BK ? kNumRecords : (uint32_t)(rem * ldb));
        k0 = ck;
        cur = rsrc_add(cur, (uint64_t)(BK * ldb));
        ck += BK;
        if constexpr (SPLIT) {
            const bool to2 = ck == split;
            cur[0] = to2 ? cur2[0] : cur[0];
            cur[1] = to2 ? cur2[1] : cur[1];
        }
        return rs;
    }
    template <bool ALIGNED>
    __device__ __forceinline__ void issue(const rsrc_t &rs, int32_t k0, int32_t red, uint32_t at, int wave,
                                          int lane, int j) const {
        (void)k0;
        (void)red;
        (void)wave;
        (void)lane;
        copy16(rs, at + j * 1024, voff[j]);
    }

    // Fragment reads (v_mfma_f32_16x16x32).  Fragment f of half ks (0, 1) of
    // a step holds columns wh * WROWS + 16 f + (lane & 15) and reduction values
    // 32 ks + 8 (lane >> 4) .. +7: two transposing reads of 4 values each
    // (rows 0..3 and 4..7 of the lane's eight), issued together.  ds_read_b64_tr_b16 hands lane j
    // of each 16 the (j % 4)-th of the 4 values read by lanes 4e + j / 4
    // (e = 0..3); pointing those lanes at 4 consecutive rows x 4 four-column
    // groups gives lane j 4 consecutive reduction values of column j.  The
    // permutation of segments depends on bits 0, 1 and 3 of k only, which
    // 32 ks + 4 t does not change, so the address is the unit's plus flo[f]
    // (fixed for the kernel) plus (32 ks + 4 t) rows of ROWB bytes (a constant).
    uint32_t flo[WROWS / 16];
    __device__ __forceinline__ void init_reads(int wh, int lane) {
        const int s = lane & 15;
        const int kl = 8 * (lane >> 4) + (s >> 2);
#pragma unroll
        for (int f = 0; f < WROWS / 16; ++f) {
            const int r = wh * WROWS + f * 16 + 4 * (s & 3);
            flo[f] = (uint32_t)(kl * ROWB + (seg_pos(kl, r >> 4) << 5) + (r & 15) * 2);
        }
    }
    // The reads of one fragment share a per-lane base, formed right before
    // them (one add) and hidden from the optimiser so that the constant parts
    // of the addresses stay in the instructions' offset fields.
    struct Bases { uint32_t unit; };
    __device__ __forceinline__ Bases bases(uint32_t unit, int ks) const {
        (void)ks;
        return Bases{unit};
    }
    __device__ __forceinline__ void frag(const Bases &b, int ks, int f, u32x4 &out) const {
        uint32_t base = b.unit + flo[f];
        asm volatile("" : "+v"(base));
        const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4 *)(uintptr_t)(base + (32 * ks) * ROWB));
        const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4 *)(uintptr_t)(base + (32 * ks + 4) * ROWB));
        const u32x2 w0 = __builtin_bit_cast(u32x2, v0), w1 = __builtin_bit_cast(u32x2, v1);
        out = u32x4{w0[0], w0[1], w1[0], w1[1]};
    }
};

// Wait until at most `n` buffer->LDS copies of this wave are in flight and all
// its LDS reads have returned, then meet the other waves.
template <int n>
__device__ __forceinline__ void wait_and_barrier() {
    static_assert(n == 6 || n == 8 || n == 10, "the pipeline keeps one unit (n copies per wave) in flight");
    if constexpr (n == 6)
        asm volatile("s_waitcnt vmcnt(6) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else if constexpr (n == 8)
        asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else
        asm volatile("s_waitcnt vmcnt(10) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ---- MFMA ------------------------------------------------------------------------

// v_mfma_f32_16x16x32: A (16 x 32) and B (32 x 16) give each lane 8 values
// (lane l: row / column l % 16, reduction values 8 (l / 16) .. +7); the 16 x 16
// fp32 result gives lane l column l % 16, rows 4 (l / 16) .. +3.  Per FLOP it
// moves half the accumulator traffic of the 32 x 32 x 16 form, and under the
// power limit it sustains ~17 % more FLOP/s on random data.
//
// Written as inline assembly with the accumulator tied to an AGPR tuple:
// with 64 small accumulators the register allocator otherwise moves them
// between registers inside the loop.  The compiler does not see these as
// MFMAs, so the wait states it would insert around them are written out
// where they matter (mfma_fence): before the accumulators are first used and
// before the epilogue reads them.  Inside the loop an accumulator feeds the
// next MFMA on the same registers directly (back-to-back chaining, which
// needs no wait states) and is then not touched for 126 MFMAs, far beyond any
// dependency latency.  The build checks the compiled code for these wait
// states.
template <typename T>
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c);

// A point that every write of the accumulators comes before and every read
// after, with more than the longest XDL-result latency of wait states
// (NOPS_FIRST: at its start, else at its end).  One volatile statement per
// accumulator (volatile statements keep their order), each tied to it.
template <bool NOPS_FIRST, int QB, int PB>
__device__ __forceinline__ void mfma_fence(f32x4 (&acc)[QB][PB]) {
    if constexpr (NOPS_FIRST) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int i = 0; i < QB; ++i)
#pragma unroll
        for (int j = 0; j < PB; ++j) asm volatile("" : "+a"(acc[i][j]));
    if constexpr (!NOPS_FIRST) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

template <>
__device__ __forceinline__ f32x4 mfma16<_Float16>(u32x4 a, u32x4 b, f32x4 c) {
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
    return c;
}

template <>
__device__ __forceinline__ f32x4 mfma16<__bf16>(u32x4 a, u32x4 b, f32x4 c) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
    return c;
}

// ---- conversions and GeLU ---------------------------------------------------------

// One round-to-nearest-even conversion (v_cvt_f16_f32 / v_cvt_pk_bf16_f32).
template <typename T>
__device__ __forceinline__ uint32_t bits16(float x) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (T)x);
}

template <typename T>
__device__ __forceinline__ float value16(uint32_t b) {
    return (float)__builtin_bit_cast(T, (uint16_t)b);
}

// GeLU(a) = a * Phi(a), Phi(a) = erfc(-a / sqrt 2) / 2 (exact erf form), in
// fp64.  The forward epilogue rounds it once to 16 bits, and its input is a
// 16-bit value, so it is a table of 65536 entries per type, built once per
// device (build_gelu_table) and looked up from LDS in the epilogue.
__device__ __forceinline__ double gelu_f64(double a) { return a * (0.5 * erfc(-a / sqrt(2.0))); }

// double -> float rounded to odd (truncate, then set the last bit if
// inexact): a later round-to-nearest-even to a format at least two bits
// narrower then gives the correctly rounded result of the double.
__device__ __forceinline__ float round_to_odd_f32(double h) {
    float f = (float)h;
    if ((double)f != h) {
        uint32_t u = __builtin_bit_cast(uint32_t, f);
        if (fabs((double)f) > fabs(h)) u -= 1;  // rounded away from zero: one step back
        f = __builtin_bit_cast(float, u | 1u);
    }
    return f;
}

__device__ uint16_t g_gelu_f16[65536];
__device__ uint16_t g_gelu_bf16[65536];

template <typename T>
__device__ __forceinline__ uint16_t *gelu_table();
template <>
__device__ __forceinline__ uint16_t *gelu_table<_Float16>() { return g_gelu_f16; }
template <>
__device__ __forceinline__ uint16_t *gelu_table<__bf16>() { return g_gelu_bf16; }

template <typename T>
__global__ __launch_bounds__(256) void gelu_table_kernel() {
    const uint32_t i = blockIdx.x * 256 + threadIdx.x;
    gelu_table<T>()[i] = (uint16_t)bits16<T>(round_to_odd_f32(gelu_f64((double)value16<T>(i))));
}

// GeLU'(a) = Phi(a) + a * phi(a), phi(a) = exp(-a^2 / 2) / sqrt(2 pi).
__device__ __forceinline__ float gelu_grad_f32(float a) {
    const float cdf = 0.5f * erfcf(-a * 0.70710678118654752f);
    const float pdf = 0.39894228040143268f * expf(-0.5f * a * a);
    return cdf + a * pdf;
}

// GeLU' in fp32 of every 16-bit input, built once per device with the
// function above (so a lookup gives the bits an evaluation would), for the
// GeLU backward.
__device__ float g_gelu_grad_f16[65536];
__device__ float g_gelu_grad_bf16[65536];

template <typename T>
__device__ __forceinline__ float *gelu_grad_table();
template <>
__device__ __forceinline__ float *gelu_grad_table<_Float16>() { return g_gelu_grad_f16; }
template <>
__device__ __forceinline__ float *gelu_grad_table<__bf16>() { return g_gelu_grad_bf16; }

template <typename T>
__global__ __launch_bounds__(256) void gelu_grad_table_kernel() {
    const uint32_t i = blockIdx.x * 256 + threadIdx.x;
    gelu_grad_table<T>()[i] = gelu_grad_f32(value16<T>(i));
}

// ---- workgroup -> macro-tile ------------------------------------------------------

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup w runs on
// XCD w % 8, as its (w / 8)-th).  XCD x is given a contiguous range of tiles,
// [x q + min(x, r), ...) of q + (x < r) tiles (nt = 8 q + r), so the
// workgroups that share an L2 also share operand tiles; inside a range, tiles
// go in column groups G macro-rows tall (G P tiles reuse one Q tile, the
// consecutive groups reuse P).  G is set per product by measurement on the
// FFN block at T = 32768: 4 for the forward and input-gradient products
// (against 8: +1-2 % each, the down-projection's forward +10 %; against 2 and
// 1: up to 2 % and 10 % slower), except 1 for the forward's 320 x 192 tiles
// (the down-projection's: forward and paired recompute 2-4 % faster than
// with 4), and 8 for the weight-gradient products (4 lost 1-2.5 %; 16 lost
// on every product).  Where G is 4 and the rows come in whole bands of 16
// macro-rows, two XCDs share each 4-row strip of a band instead (the first
// and second half of its column-major order), so that a round of workgroups
// touches 16 row panels and 17 column panels rather than 32 and 8: the
// up-projection's forward, whose round of panels (13 MB each) exceeds the
// 256 MB Infinity Cache, ran 2.2 % faster, the dX products the same.  With
// G = 8 (the weight-gradient products) all XCDs work in the same group at
// once, each on an eighth of it (8 rows x tiles_q / 8 columns), so that a
// round touches 8 row panels instead of all of them: the up-projection's dW
// (25 x 100 tiles of 256, panels of 16.8 MB) ran 1.2-2.0 % faster.  With
// G = 1 and an even number of column tiles (the down-projection's recompute
// over two weight tiles), the left half of the columns comes first, so that
// XCDs 0-3 read only the first tile's panels and 4-7 only the second's
// (6.4 rows x 5 columns each instead of 3.2 x 10: a quarter fewer L2 misses
// per round, the same HBM bytes): that launch ran 1.4 % faster.
template <int G>
__device__ __forceinline__ void tile_coords(int w, int tiles_p, int tiles_q, int &tp, int &tq) {
    const int nt = tiles_p * tiles_q;
    const int x = w & 7, k = w >> 3;
    if constexpr (G == 4) {
        if ((tiles_p & 15) == 0) {
            // bands of 16 macro-rows, each 4 strips of 4 rows in column-major
            // order; XCDs 2s and 2s + 1 take the first and second half of strip
            // s of every band, each its k-th tile of the band at position k
            const int per = 2 * tiles_q;
            const int band = k / per;
            const int pos = (x & 1) * per + (k - band * per);
            tp = band * 16 + (x >> 1) * 4 + (pos & 3);
            tq = pos >> 2;
            return;
        }
    }
    if constexpr (G == 1) {
        if ((tiles_q & 1) == 0) {
            // the left half of the columns first, then the right half (a
            // product over two weight tiles: XCDs 0-3 on the first tile,
            // 4-7 on the second, each reading half the weight panels)
            const int q8 = nt >> 3, r8 = nt & 7;
            const int t = x * q8 + min(x, r8) + k;
            const int hq = tiles_q >> 1, half = tiles_p * hq;
            const int h = t >= half ? 1 : 0;
            const int r = t - h * half;
            tp = r / hq;
            tq = h * hq + (r - (r / hq) * hq);
            return;
        }
    }
    if constexpr (G == 8) {
        // every XCD in the same 8-row group at once, XCD x on the x-th eighth
        // of its column-major order (tiles_q tiles each); the rows left below
        // the last full group split by contiguous ranges as below
        const int full = tiles_p >> 3;
        if (k < full * tiles_q) {
            const int g = k / tiles_q;
            const int pos = x * tiles_q + (k - g * tiles_q);
            tp = g * 8 + (pos & 7);
            tq = pos >> 3;
        } else {
            const int rows = tiles_p - 8 * full;
            const int n = rows * tiles_q;
            const int pos = x * (n >> 3) + min(x, n & 7) + (k - full * tiles_q);
            tp = full * 8 + pos % rows;
            tq = pos / rows;
        }
        return;
    }
    const int q8 = nt >> 3, r8 = nt & 7;
    const int t = x * q8 + min(x, r8) + k;
    const int per_group = G * tiles_q;
    const int g = t / per_group;
    const int first = g * G;
    const int gsz = min(tiles_p - first, G);
    const int r = t - g * per_group;
    tp = first + r % gsz;
    tq = r / gsz;
}

// ---- the GEMM ---------------------------------------------------------------------

// f(integral_constant<int, I>) for I = B .. E-1, unrolled by construction (a
// large loop body can exceed the unroller's size limit, and a rolled loop
// would index the accumulators at run time).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

template <bool RS, int ROWS>
using OperandT = typename std::conditional<RS, RsOperand<ROWS>, RcOperand<ROWS>>::type;

// Position of copy k of the first half of a step's MFMAs (n copies spread
// evenly over MFMAs 0 .. half - 1): MFMA (half (2 k + 1)) / (2 n).  Returns
// the k whose copy follows MFMA m, or -1.
template <int n, int half>
__device__ constexpr int copy_at(int m) {
    for (int k = 0; k < n; ++k)
        if ((half * (2 * k + 1)) / (2 * n) == m) return k;
    return -1;
}

// The macro-tile is (32 QB) columns of q by (32 PB) rows of p; each of the
// four waves owns a (16 QB) x (16 PB) quarter: QB x PB blocks of 16 x 16, so
// 4 QB PB fp32 accumulators per lane (at most 256: one wave per SIMD).
//   (8, 8)   256 x 256, every product;
//   (10, 6)  320 x 192, forward products whose q extent (the tile width) is
//            a multiple of 320 but not of 256 (the down-projection's 1600);
//   (6, 10)  192 x 320, gradient products whose p extent is such a width.
// PERSIST (accumulating products only): a workgroup takes the output tiles
// of workgroup indices w, w + G, w + 2G, ... (G = the grid, a multiple of 8,
// so all of them fall on the XCD of w and keep its tile order); between two
// tiles the next one's first operand units are copied and its C loaded while
// the finished one's accumulators are stored.
template <typename T, bool Q_RS, bool P_RS, int EPI, bool ALIGNED, int QB, int PB, bool PERSIST>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_kernel(GemmArgs a, int tiles_p, int tiles_q) {
    constexpr int TQ = 32 * QB, TP = 32 * PB;
    static_assert(QB * PB <= 64, "accumulators beyond the 256 AGPRs of a lane");
    static_assert((EPI != EPI_ACC && EPI != EPI_GELU && EPI != EPI_GELU_F32A) || (QB == 8 && PB == 8),
                  "the accumulating and GeLU epilogues are built for the 256 x 256 tile");
    static_assert(!PERSIST || EPI == EPI_ACC, "only the accumulating product runs persistent workgroups");
    using QOp = OperandT<Q_RS, TQ>;
    using POp = OperandT<P_RS, TP>;
    // LDS ring.  Each step's two units are issued first-operand first; the
    // pipeline keeps three first-operand units and two second-operand units
    // alive (see the main loop), so the operand with the smaller unit goes
    // first.  Equal units share one ring of five slots.
    constexpr bool Q_FIRST = QOp::UNIT <= POp::UNIT;
    constexpr int UF = Q_FIRST ? QOp::UNIT : POp::UNIT;
    constexpr int US = Q_FIRST ? POp::UNIT : QOp::UNIT;
    constexpr int NF = Q_FIRST ? QOp::NCOPY : POp::NCOPY;  // copies per wave of a first-operand unit
    constexpr int NS = Q_FIRST ? POp::NCOPY : QOp::NCOPY;
    constexpr bool MIXED = UF == US;
    constexpr int LDS_BYTES = MIXED ? 5 * UF : 3 * UF + 2 * US;
    static_assert(LDS_BYTES <= 160 * 1024, "the ring exceeds the LDS");
    static_assert(EPI != EPI_GELU && EPI != EPI_GELU_F32A ? true : LDS_BYTES >= 65536 * 2, "GeLU table");
    __shared__ __attribute__((aligned(1024))) char lds[LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wq = wave & 1;
    const int wp = wave >> 1;

    int w = blockIdx.x;  // workgroup index of the current output tile
    int64_t p0, q0;      // its first output row and column
    // GeLU forward: the last split_tail tiles of the launch are each taken by
    // two workgroups, one half of the reduction each (workgroups from index
    // tiles - split_tail on, two per tile); half < 0 for a whole tile.
    constexpr bool GELU = EPI == EPI_GELU || EPI == EPI_GELU_F32A;
    int half = -1, sj = 0;
    if constexpr (GELU) {
        const int first = tiles_p * tiles_q - a.split_tail;
        if (w >= first) {
            sj = (w - first) >> 1;
            half = (w - first) & 1;
            w = first + sj;
        }
    }
    QOp qo;
    POp po;
    // The operands of the output tile of workgroup index wi, their copy
    // cursors at the first step.  (ln is the lane index; a persistent
    // workgroup passes it through an opaque copy, so that the per-lane
    // offsets are formed anew for each tile rather than kept, or spilled,
    // across the main loop.)
    auto setup = [&](int wi, int ln) __attribute__((always_inline)) {
        int tp, tq;
        tile_coords<(Q_RS && P_RS) ? 8 : (QB == 10 ? 1 : 4)>(wi, tiles_p, tiles_q, tp, tq);
        p0 = (int64_t)tp * TP;
        q0 = (int64_t)tq * TQ;
        if constexpr (Q_RS) {
            qo.init(static_cast<const uint16_t *>(a.Q), a.ldq, q0, a.cols, wave, ln);
            qo.set_split(a.Q2, a.qsplit, q0);
        } else {
            // a forward product over two weight tiles: columns from qsplit on
            // are rows of Q2 (qsplit is a multiple of the macro-tile's width, so
            // a workgroup reads one tile)
            const bool second = a.Q2 && q0 >= a.qsplit;
            qo.init(static_cast<const uint16_t *>(second ? a.Q2 : a.Q), a.ldq, second ? q0 - a.qsplit : q0,
                    second ? a.cols - a.qsplit : a.cols, wave, ln);
        }
        po.init(static_cast<const uint16_t *>(a.P), a.ldp, p0, a.rows, wave, ln);
        qo.init_cursor();
        po.init_cursor();
    };
    setup(w, lane);
    if constexpr (GELU) {
        static_assert(!Q_RS && !P_RS, "a split half offsets reduction-contiguous rows");
        if (half > 0) {  // the second half of the reduction
            const int64_t koff = (a.red >> 1) * 2;
            qo.base += koff;
            po.base += koff;
            qo.init_cursor();
            po.init_cursor();
        }
    }
    qo.init_reads(wq, lane);
    po.init_reads(wp, lane);

    // Operand units: the first operand of step s is unit 2s, the second unit
    // 2s + 1.  Copies and fragment reads are spread evenly between the
    // MFMAs, so that no wave stalls on a burst of copies while its matrix
    // unit idles.
    // below 2^30 (the host checks); a split half runs half of it, a whole
    // number of steps (the host checks)
    const int32_t red = (int32_t)(half >= 0 ? a.red >> 1 : a.red);
    const int64_t ksteps = (red + BK - 1) / BK;
    // slot of unit u (used for the first five units; the ring below rotates
    // from there)
    auto slot = [&](int u) __attribute__((always_inline)) -> char * {
        if constexpr (MIXED) {
            return lds + (u % 5) * UF;
        } else {
            const int st = u >> 1;
            return (u & 1) ? lds + 3 * UF + (st & 1) * US : lds + (st % 3) * UF;
        }
    };
    // The next step of the first / second operand to copy (in step order).
    constexpr bool SPLIT = EPI == EPI_ACC;  // only the input-gradient product splits its reduction over two tiles
    auto take_f = [&](int32_t &k0) __attribute__((always_inline)) -> rsrc_t {
        if constexpr (Q_FIRST) return qo.template take<ALIGNED, SPLIT>(red, k0);
        else return po.template take<ALIGNED, false>(red, k0);
    };
    auto take_s = [&](int32_t &k0) __attribute__((always_inline)) -> rsrc_t {
        if constexpr (Q_FIRST) return po.template take<ALIGNED, false>(red, k0);
        else return qo.template take<ALIGNED, SPLIT>(red, k0);
    };
    // copy j of such a step into the unit at LDS address `unit`
    const uint32_t wf = (uint32_t)(wave * NF * 1024), ws = (uint32_t)(wave * NS * 1024);
    auto issue_f = [&](const rsrc_t &rs, int32_t k0, uint32_t unit, int j) __attribute__((always_inline)) {
        if constexpr (Q_FIRST) qo.template issue<ALIGNED>(rs, k0, red, unit + wf, wave, lane, j);
        else po.template issue<ALIGNED>(rs, k0, red, unit + wf, wave, lane, j);
    };
    auto issue_s = [&](const rsrc_t &rs, int32_t k0, uint32_t unit, int j) __attribute__((always_inline)) {
        if constexpr (Q_FIRST) po.template issue<ALIGNED>(rs, k0, red, unit + ws, wave, lane, j);
        else qo.template issue<ALIGNED>(rs, k0, red, unit + ws, wave, lane, j);
    };

    using QBs = typename QOp::Bases;
    using PBs = typename POp::Bases;

    // acc[i][j]: the 16 x 16 block of q-block i and p-block j of this wave.
    // Register e of block (i, j) holds C[p][q] with
    // p = p0 + wp 16 PB + 16 j + (lane & 15), q = q0 + wq 16 QB + 16 i + 4 (lane >> 4) + e.
    // An accumulating product starts from C, so its epilogue is a plain
    // store.  C is loaded straight into the accumulator registers (every
    // lane, every block: out-of-range elements, and all of them when not
    // accumulating, come back as zeros from the buffer unit), issued before
    // the first operand copies, so the prologue's wait for the first two
    // steps' units (vmcnt counts loads in issue order) covers it too.  Row
    // block j has its own descriptor, so a lane offset stays below
    // 16 ldc + 256 elements (the host keeps that under the descriptor's range).
    // c_rsrc / c_off: that descriptor (records = 0: every read gives zero) and
    // this lane's offset of block (i, j) in the tile at (p0_, q0_), kOOB
    // outside C (a load reads zero there and a store is dropped).
    auto c_rsrc = [&](int64_t p0_, int64_t q0_, int j, bool live) __attribute__((always_inline)) -> rsrc_t {
        const int64_t prow = p0_ + wp * (16 * PB) + 16 * j;
        return make_rsrc(reinterpret_cast<const char *>(static_cast<const float *>(a.C) + prow * a.ldc + q0_),
                         live ? kNumRecords : 0u);
    };
    auto c_off = [&](int64_t p0_, int64_t q0_, int i, int j, int ln) __attribute__((always_inline)) -> uint32_t {
        const int64_t p = p0_ + wp * (16 * PB) + (ln & 15) + 16 * j;
        const int64_t q = q0_ + wq * (16 * QB) + 4 * (ln >> 4) + 16 * i;
        return (p < a.rows && q < a.cols) ? (uint32_t)(((ln & 15) * a.ldc + (q - q0_)) * 4) : kOOB;
    };
    f32x4 acc[QB][PB];
#pragma unroll
    for (int j = 0; j < PB; ++j) {
        if constexpr (EPI == EPI_ACC) {
            const rsrc_t rs = c_rsrc(p0, q0, j, a.accumulate != 0);
#pragma unroll
            for (int i = 0; i < QB; ++i)
                asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen"
                             : "=a"(acc[i][j])
                             : "v"(c_off(p0, q0, i, j, lane)), "s"(rs)
                             : "memory");
        } else {
#pragma unroll
            for (int i = 0; i < QB; ++i) acc[i][j] = f32x4{};
        }
    }

    // Fragments of one step (64 reduction values in two halves h = 0, 1).
    // The MFMAs of a step run over the blocks row by row of the "row"
    // operand (the one with more blocks per wave; Q on a tie) and, within a
    // row, over the blocks of the "column" operand.  Block (i, j) takes its
    // two MFMAs back to back (h = 0, then h = 1), so the matrix core chains
    // the second onto the first through its accumulator without a
    // register-file round trip, which saves power (and so clock) under the
    // board's limit.  A row operand fragment is dead after its row's last
    // MFMA, so the next step's fragments of that row are read into the same
    // registers right after it; its last row and every column-operand
    // fragment are used to the end of the step and are double-buffered
    // (parity `par` of the step).  Column reads are spread over the first
    // part of the step.
    constexpr bool ROW_Q = QB >= PB;
    constexpr int NR = ROW_Q ? QB : PB;  // rows of blocks
    constexpr int NC = ROW_Q ? PB : QB;  // blocks per row
    constexpr int NM = 2 * NR * NC;      // MFMAs per step
    constexpr int MH = NM / 2;
    u32x4 xr[NR - 1][2], xrl[2][2], xc[2][NC][2];
    auto qfrag = [&](const QBs &b0, const QBs &b1, int h, int f, u32x4 &out) __attribute__((always_inline)) {
        qo.frag(h ? b1 : b0, h, f, out);
    };
    auto pfrag = [&](const PBs &b0, const PBs &b1, int h, int f, u32x4 &out) __attribute__((always_inline)) {
        po.frag(h ? b1 : b0, h, f, out);
    };
    // One step: NM MFMAs; between them the reads of the next step (at the
    // bases qb0, qb1, pb0, pb1) and the copies: copy_a(0 .. NS-1) in the
    // first half, copy_b(0 .. NF-1) in the second.
    auto step = [&](auto PAR, const QBs &qb0, const QBs &qb1, const PBs &pb0, const PBs &pb1, auto &&copy_a,
                    auto &&copy_b) __attribute__((always_inline)) {
        constexpr int par = decltype(PAR)::value;
        auto rfrag = [&](int h, int f, u32x4 &out) __attribute__((always_inline)) {
            if constexpr (ROW_Q) qfrag(qb0, qb1, h, f, out); else pfrag(pb0, pb1, h, f, out);
        };
        auto cfrag = [&](int h, int f, u32x4 &out) __attribute__((always_inline)) {
            if constexpr (ROW_Q) pfrag(pb0, pb1, h, f, out); else qfrag(qb0, qb1, h, f, out);
        };
        static_for<0, NM>([&](auto M_) __attribute__((always_inline)) {
            constexpr int m = decltype(M_)::value;
            constexpr int blk = m >> 1, h = m & 1, r = blk / NC, c = blk % NC;
            constexpr int i = ROW_Q ? r : c, j = ROW_Q ? c : r;
            u32x4 &rf = (r < NR - 1) ? xr[r < NR - 1 ? r : 0][h] : xrl[par][h];
            u32x4 &cf = xc[par][c][h];
            (void)i;
            (void)j;
            acc[i][j] = mfma16<T>(ROW_Q ? rf : cf, ROW_Q ? cf : rf, acc[i][j]);
            if constexpr (m % 4 == 1 && m < 8 * NC) {  // column fragment (m / 8, (m / 4) % 2) of the next step
                constexpr int f = m / 8, hh = (m / 4) & 1;
                cfrag(hh, f, xc[par ^ 1][f][hh]);
            }
            if constexpr ((m + 1) % (2 * NC) == 0 && m / (2 * NC) < NR - 1) {  // row m / (2 NC) of the next step
                constexpr int row = m / (2 * NC);
                rfrag(0, row, xr[row][0]);
                rfrag(1, row, xr[row][1]);
            }
            if constexpr (m == MH + 2) rfrag(0, NR - 1, xrl[par ^ 1][0]);
            if constexpr (m == MH + 6) rfrag(1, NR - 1, xrl[par ^ 1][1]);
            if constexpr (m < MH) {
                constexpr int k = copy_at<NS, MH>(m);
                if constexpr (k >= 0) copy_a(k);
            } else {
                constexpr int k = copy_at<NF, MH>(m - MH);
                if constexpr (k >= 0) copy_b(k);
            }
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;

    // The slot ring: rg[k] is the LDS address of the slot of unit 2s + k
    // (k = 0 .. 4) at step s.  Step s reads units 2s + 2 and 2s + 3, and
    // copies unit 2s + 5 into the slot of unit 2s + 1 (with equal units, of
    // unit 2s: (2s + 5) mod 5 = 2s mod 5) and unit 2s + 6 into that of unit
    // 2s (of unit 2s + 1); both were read during step s - 1.  Moving on a step
    // shifts the ring by two units and appends those two slots.
    uint32_t rg[5];

    // Prologue: units 0..4 in flight (units past the last one read zeros);
    // wait for units 0..3, read the fragments of step 0.
    auto copy_first_units = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < 5; ++k) rg[k] = lds_addr(slot(k));
        static_for<0, 5>([&](auto U_) __attribute__((always_inline)) {
            constexpr int u = decltype(U_)::value;
            int32_t k0;
            if constexpr (u % 2 == 0) {
                const rsrc_t rs = take_f(k0);
#pragma unroll
                for (int j = 0; j < NF; ++j) issue_f(rs, k0, rg[u], j);
            } else {
                const rsrc_t rs = take_s(k0);
#pragma unroll
                for (int j = 0; j < NS; ++j) issue_s(rs, k0, rg[u], j);
            }
        });
    };
    auto read_first_fragments = [&]() __attribute__((always_inline)) {
        const uint32_t qs = Q_FIRST ? rg[0] : rg[1], ps = Q_FIRST ? rg[1] : rg[0];
        const QBs qb0 = qo.bases(qs, 0), qb1 = qo.bases(qs, 1);
        const PBs pb0 = po.bases(ps, 0), pb1 = po.bases(ps, 1);
#pragma unroll
        for (int f = 0; f < NR; ++f)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                u32x4 &dst = f < NR - 1 ? xr[f < NR - 1 ? f : 0][h] : xrl[0][h];
                if constexpr (ROW_Q) qfrag(qb0, qb1, h, f, dst); else pfrag(pb0, pb1, h, f, dst);
            }
#pragma unroll
        for (int f = 0; f < NC; ++f)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if constexpr (ROW_Q) pfrag(pb0, pb1, h, f, xc[0][f][h]); else qfrag(qb0, qb1, h, f, xc[0][f][h]);
            }
    };
    copy_first_units();
    wait_and_barrier<NF>();
    read_first_fragments();

    // Read bases of the next step (units 2s + 2, 2s + 3), formed before the
    // barrier that precedes the step, so that the step opens with its MFMAs.
    QBs qb0, qb1;
    PBs pb0, pb1;
    auto next_bases = [&]() __attribute__((always_inline)) {
        const uint32_t qs = Q_FIRST ? rg[2] : rg[3], ps = Q_FIRST ? rg[3] : rg[2];
        qb0 = qo.bases(qs, 0);
        qb1 = qo.bases(qs, 1);
        pb0 = po.bases(ps, 0);
        pb1 = po.bases(ps, 1);
    };
    next_bases();

    mfma_fence<false>(acc);  // accumulator writes, then the first MFMA

    // Step s reads step s + 1 from units 2s + 2, 2s + 3 (landed), copies unit
    // 2s + 5 (the second operand of step s + 2) under its first half and unit
    // 2s + 6 (the first operand of step s + 3) under its second half; at its
    // end every wave has read units 2s + 2, 2s + 3, and units 2s + 4 and
    // 2s + 5 must have landed (unit 2s + 6 may still be in flight: NF copies
    // per wave).
    auto one_step = [&](auto PAR) __attribute__((always_inline)) {
        const uint32_t ca = MIXED ? rg[0] : rg[1];  // unit 2s + 5
        const uint32_t cb = MIXED ? rg[1] : rg[0];  // unit 2s + 6
        rsrc_t rsa, rsb;
        int32_t ka, kb;
        step(PAR, qb0, qb1, pb0, pb1,
             [&](int c) __attribute__((always_inline)) {
                 if (c == 0) rsa = take_s(ka);
                 issue_s(rsa, ka, ca, c);
             },
             [&](int c) __attribute__((always_inline)) {
                 if (c == 0) rsb = take_f(kb);
                 issue_f(rsb, kb, cb, c);
             });
        const uint32_t r2 = rg[2], r3 = rg[3], r4 = rg[4];
        rg[0] = r2;
        rg[1] = r3;
        rg[2] = r4;
        rg[3] = ca;
        rg[4] = cb;
        next_bases();
    };

    // Every MFMA sits in this loop, whose body is two steps (the register
    // parity).  With an odd step count its last pass runs one step past the
    // end, on fragments read from units past the last one: zeros, which add
    // nothing.  A tail outside the loop would let the register allocator
    // place accumulator copies between the MFMAs, which it cannot see as such
    // and so would not separate by the wait states they need.  The barrier
    // between two steps opens the body rather than closing it, so that the
    // register moves of the loop's back edge fall before it, under the last
    // MFMAs, and every step starts with its first MFMA.  (Before the first
    // step it finds everything it waits for already done.)
    const int64_t npairs = (ksteps + 1) / 2;
    for (;;) {  // one pass per output tile of this workgroup
        for (int64_t t = 0; t < npairs; ++t) {
            wait_and_barrier<NF>();
            one_step(P0{});
            wait_and_barrier<NF>();
            one_step(P1{});
        }
        mfma_fence<true>(acc);  // the last MFMA, then accumulator reads
        // the copies past the last unit are still in flight: none may land
        // after the workgroup has released its LDS, or under the next tile's
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        if constexpr (PERSIST) {
            const int wn = w + (int)gridDim.x;
            if (wn < tiles_p * tiles_q) {
                const int64_t pd = p0, qd = q0;  // the finished tile
                // every wave has read its last fragments before the ring refills
                asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
                int ln = lane;
                asm volatile("" : "+v"(ln));
                w = wn;
                setup(w, ln);
                copy_first_units();
                // Store the finished tile's sums, then load the next tile's C
                // into the same registers (a store reads its data registers
                // when it issues, so no load can overtake it).  All stores go
                // out before the first load: interleaved, the two took about
                // a tenth longer.
#pragma unroll
                for (int j = 0; j < PB; ++j) {
                    const rsrc_t rst = c_rsrc(pd, qd, j, true);
#pragma unroll
                    for (int i = 0; i < QB; ++i)
                        asm volatile("buffer_store_dwordx4 %0, %1, %2, 0 offen"
                                     : "+a"(acc[i][j])
                                     : "v"(c_off(pd, qd, i, j, ln)), "s"(rst)
                                     : "memory");
                }
#pragma unroll
                for (int j = 0; j < PB; ++j) {
                    const rsrc_t rld = c_rsrc(p0, q0, j, a.accumulate != 0);
#pragma unroll
                    for (int i = 0; i < QB; ++i)
                        asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen"
                                     : "+a"(acc[i][j])
                                     : "v"(c_off(p0, q0, i, j, ln)), "s"(rld)
                                     : "memory");
                }
                asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
                read_first_fragments();
                next_bases();
                mfma_fence<false>(acc);  // accumulator writes, then the first MFMA
                continue;
            }
        }
        break;
    }

    // A split half stores its fp32 sums, in the accumulators' own layout
    // (each lane's 16 bytes of a block side by side: 1 KiB per wave and
    // block), and counts itself in; the half that arrives second adds the
    // other's sums in the epilogue and finishes the tile, and the first ends
    // here.  Neither waits for the other.  The sum of the two halves does
    // not depend on which arrives second.
    const f32x4 *other = nullptr;
    if constexpr (GELU) {
        if (half >= 0) {
            constexpr int kWave = QB * PB * 64;  // a wave's share of a half: f32x4 each
            f32x4 *part = reinterpret_cast<f32x4 *>(a.split_part);
            f32x4 *mine = part + ((int64_t)(2 * sj + half) * 4 + wave) * kWave + lane;
#pragma unroll
            for (int i = 0; i < QB; ++i)
#pragma unroll
                for (int j = 0; j < PB; ++j) mine[(i * PB + j) * 64] = acc[i][j];
            __threadfence();  // the sums reach device scope before the count
            // every wave's sums stored and its reads of the ring returned:
            // the first word of LDS then carries the count to the waves
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            volatile uint32_t *word = reinterpret_cast<volatile uint32_t *>(lds);
            if (tid == 0) *word = atomicAdd(a.split_cnt + sj, 1u);
            __syncthreads();
            if (*word == 0) return;  // the other half finishes this tile
            if (tid == 0) atomicExch(a.split_cnt + sj, 0u);  // zero again for the next launch
            __threadfence();  // the other half's sums are read after its count
            other = part + ((int64_t)(2 * sj + (1 - half)) * 4 + wave) * kWave + lane;
        }
    }

    // Epilogue.
    const int64_t pb = p0 + wp * (16 * PB) + (lane & 15);
    const int64_t qb = q0 + wq * (16 * QB) + 4 * (lane >> 4);
    if constexpr (EPI == EPI_GELU || EPI == EPI_GELU_F32A) {
        // H = table[A]: the GeLU table of this type goes into the now idle LDS
        // (128 KiB: 32 one-KiB copies per wave).  Every wave's copies of the
        // main loop must have landed, and every wave's reads of the ring
        // returned, before the table overwrites the ring.
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        const rsrc_t rs = make_rsrc(reinterpret_cast<const char *>(gelu_table<T>()), 65536u * 2u);
#pragma unroll
        for (int c = 0; c < 32; ++c) {
            const int blk = wave * 32 + c;
            copy16(rs, lds_addr(lds + blk * 1024), (uint32_t)(blk * 1024 + lane * 16));
        }
        asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    }
    [[maybe_unused]] const __attribute__((address_space(3))) uint16_t *gtab =
        (const __attribute__((address_space(3))) uint16_t *)(uintptr_t)lds_addr(lds);
#pragma unroll
    for (int i = 0; i < QB; ++i) {
        const int64_t q = qb + i * 16;
        if (q >= a.cols) continue;
#pragma unroll
        for (int j = 0; j < PB; ++j) {
            const int64_t p = pb + j * 16;
            if (p >= a.rows) continue;
            f32x4 v = acc[i][j];
            if constexpr (GELU) {
                if (other) {
                    const f32x4 o = other[(i * PB + j) * 64];
                    v = f32x4{v[0] + o[0], v[1] + o[1], v[2] + o[2], v[3] + o[3]};
                }
            }
            const int64_t off = p * a.ldc + q;
            if constexpr (EPI == EPI_F32 || EPI == EPI_ACC) {
                *reinterpret_cast<f32x4 *>(static_cast<float *>(a.C) + off) = v;
            } else if constexpr (EPI == EPI_LP) {
                u32x2 o = {bits16<T>(v[0]) | (bits16<T>(v[1]) << 16), bits16<T>(v[2]) | (bits16<T>(v[3]) << 16)};
                *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(a.C) + off) = o;
            } else {  // A = RNE(acc) (or acc itself in fp32); H = RNE(GeLU(RNE(acc))) from the table
                uint32_t b[4], h[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    b[e] = bits16<T>(v[e]);
                    h[e] = gtab[b[e]];
                }
                if constexpr (EPI == EPI_GELU)
                    *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(a.C) + off) =
                        u32x2{b[0] | (b[1] << 16), b[2] | (b[3] << 16)};
                else
                    *reinterpret_cast<f32x4 *>(static_cast<float *>(a.C) + off) = v;
                *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(a.C2) + off) =
                    u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
            }
        }
    }
}

// ---- dA = RNE(dH * GeLU'(A)) ----------------------------------------------------------

// dA = RNE(dH * GeLU'(A)) with GeLU' looked up rather than evaluated: the
// evaluation (erfc and exp, tens of instructions per element) held the
// kernel at half the HBM rate.  A workgroup of 1024 threads (one per compute
// unit, with its LDS) copies the table's entries for |A| < 16 (both signs,
// kLim codes each: 152 KiB for fp16, 131 KiB for bf16) into LDS and reads the
// rest, which Gaussian-like data almost never holds, from the global table.
// OUT_F32: dA is written as the fp32 product itself, the value the 16-bit
// form rounds once.
template <typename T>
constexpr uint32_t gelu_grad_lim() { return std::is_same<T, _Float16>::value ? 0x4C00u : 0x4180u; }  // code of 16.0

template <typename T, bool OUT_F32>
__global__ __launch_bounds__(1024) void gelu_bwd_kernel(const float *__restrict__ dH,
                                                        const uint16_t *__restrict__ A,
                                                        void *__restrict__ dA, int64_t count) {
    constexpr uint32_t kLim = gelu_grad_lim<T>();
    static_assert(kLim % 4 == 0 && 2 * kLim * 4 <= 160 * 1024, "LDS table");
    __shared__ __attribute__((aligned(16))) float tab[2 * kLim];
    const float *gtab = gelu_grad_table<T>();
    for (uint32_t e = threadIdx.x * 4; e < 2 * kLim; e += blockDim.x * 4) {  // codes [0, kLim), [0x8000, +kLim)
        const uint32_t c = e < kLim ? e : 0x8000u + (e - kLim);
        *reinterpret_cast<f32x4 *>(tab + e) = *reinterpret_cast<const f32x4 *>(gtab + c);
    }
    __syncthreads();
    auto grad = [&](uint32_t c) __attribute__((always_inline)) -> float {
        const uint32_t m = c & 0x7fffu;
        return m < kLim ? tab[(c >> 15) * kLim + m] : gtab[c];
    };
    const int64_t stride = (int64_t)gridDim.x * blockDim.x * 8;
    uint16_t *dA16 = static_cast<uint16_t *>(dA);
    float *dA32 = static_cast<float *>(dA);
    for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8; i < count; i += stride) {
        if (i + 8 <= count) {
            const f32x4 g0 = *reinterpret_cast<const f32x4 *>(dH + i);
            const f32x4 g1 = *reinterpret_cast<const f32x4 *>(dH + i + 4);
            const u32x4 av = *reinterpret_cast<const u32x4 *>(A + i);
            const float g[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
            float r[8];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                r[2 * w] = g[2 * w] * grad(av[w] & 0xffffu);
                r[2 * w + 1] = g[2 * w + 1] * grad(av[w] >> 16);
            }
            // the product is rounded to fp32 first and then, once, to 16 bits:
            // kept from fusing into a mixed-precision multiply that would
            // round the exact product straight to 16 bits
#pragma unroll
            for (int e = 0; e < 8; ++e) asm volatile("" : "+v"(r[e]));
            if constexpr (OUT_F32) {
                *reinterpret_cast<f32x4 *>(dA32 + i) = f32x4{r[0], r[1], r[2], r[3]};
                *reinterpret_cast<f32x4 *>(dA32 + i + 4) = f32x4{r[4], r[5], r[6], r[7]};
            } else {
                u32x4 o;
#pragma unroll
                for (int w = 0; w < 4; ++w) o[w] = bits16<T>(r[2 * w]) | (bits16<T>(r[2 * w + 1]) << 16);
                *reinterpret_cast<u32x4 *>(dA16 + i) = o;
            }
        } else {
            for (int64_t e = i; e < count; ++e) {
                float r = dH[e] * grad(A[e]);
                asm volatile("" : "+v"(r));
                if constexpr (OUT_F32)
                    dA32[e] = r;
                else
                    dA16[e] = (uint16_t)bits16<T>(r);
            }
        }
    }
}

// Launch shapes (per-wave blocks of q, p).  A product takes the 256 x 256
// tile unless a 320-wide tile covers its tile width (the forward's q extent,
// the gradient's p extent) with clearly less padding: the down-projection's
// 1600-column tiles fill 6.25 tiles of 256 but exactly 5 of 320.  (A 320 x 128
// forward tile, which at T = 32768 would fill five whole rounds of workgroups
// on 256 compute units where 320 x 192 leaves the fourth a third full, ran
// 14 % slower: 80 MFMAs per step do not cover the step's barrier and copies.)
enum Shape { SHAPE_8x8 = 0, SHAPE_10x6 = 1, SHAPE_6x10 = 2 };

int64_t padded(int64_t x, int64_t t) { return (x + t - 1) / t * t; }

Shape shape_for(GemmOp op, int64_t rows, int64_t cols) {
    const int64_t a88 = padded(cols, 256) * padded(rows, 256);
    if (op == GemmOp::Fwd) {
        const int64_t a = padded(cols, 320) * padded(rows, 192);
        if (a * 50 < a88 * 49) return SHAPE_10x6;
    } else if (op == GemmOp::Dw) {
        const int64_t a = padded(cols, 192) * padded(rows, 320);
        if (a * 50 < a88 * 49) return SHAPE_6x10;
    }
    return SHAPE_8x8;
}

template <typename T, bool Q_RS, bool P_RS, int EPI, int QB, int PB>
hipError_t run_shape(const GemmArgs &a, hipStream_t s) {
    const int tiles_p = (int)((a.rows + 32 * PB - 1) / (32 * PB));
    const int tiles_q = (int)((a.cols + 32 * QB - 1) / (32 * QB));
    const int64_t nt = (int64_t)tiles_p * tiles_q;
    if (nt <= 0) return hipSuccess;
    // the kernel counts reduction indices in 32 bits
    if (a.red < 1 || a.red >= ((int64_t)1 << 30)) return hipErrorInvalidValue;
    // a second weight tile: reduction rows from qsplit on (gradient products),
    // or output columns from qsplit on (forward products), which no
    // workgroup's columns may straddle
    if (a.Q2) {
        if (Q_RS && (a.qsplit <= 0 || a.qsplit % BK != 0 || a.qsplit >= a.red)) return hipErrorInvalidValue;
        if (!Q_RS && (a.qsplit <= 0 || a.qsplit % (32 * QB) != 0 || a.qsplit >= a.cols)) return hipErrorInvalidValue;
    }
    // the accumulating epilogue addresses 16 rows of C through one descriptor
    if (EPI == EPI_ACC && (a.ldc < 0 || (16 * a.ldc + 256) * 4 >= (int64_t)kNumRecords)) return hipErrorInvalidValue;
    // persistent workgroups: a grid of wg_cap (a multiple of 8, so that each
    // workgroup's tiles stay on its XCD) when there are more tiles than that
    if (a.wg_cap < 0 || a.wg_cap % 8 != 0) return hipErrorInvalidValue;
    if constexpr (EPI == EPI_ACC) {
        if (a.wg_cap > 0 && nt > a.wg_cap) {
            const dim3 g((unsigned)a.wg_cap);
            if (a.red % BK == 0)
                hipLaunchKernelGGL((gemm_kernel<T, Q_RS, P_RS, EPI, true, QB, PB, true>), g, dim3(kThreads), 0, s, a,
                                   tiles_p, tiles_q);
            else
                hipLaunchKernelGGL((gemm_kernel<T, Q_RS, P_RS, EPI, false, QB, PB, true>), g, dim3(kThreads), 0, s,
                                   a, tiles_p, tiles_q);
            return hipGetLastError();
        }
    }
    // GeLU forward: when the last round of tiles would leave at least half
    // of the compute units idle, its tiles run as two half-reductions each
    GemmArgs b = a;
    b.split_tail = 0;
    if constexpr (EPI == EPI_GELU || EPI == EPI_GELU_F32A) {
        if (a.split_part && a.split_cnt && a.split_cap > 0 && a.red % (2 * BK) == 0) {
            const int64_t r = nt % a.split_cap;
            if (r > 0 && 2 * r <= a.split_cap && r <= kSplitTiles) b.split_tail = (int32_t)r;
        }
    }
    const dim3 g((unsigned)(nt + b.split_tail));
    if (a.red % BK == 0)
        hipLaunchKernelGGL((gemm_kernel<T, Q_RS, P_RS, EPI, true, QB, PB, false>), g, dim3(kThreads), 0, s, b,
                           tiles_p, tiles_q);
    else
        hipLaunchKernelGGL((gemm_kernel<T, Q_RS, P_RS, EPI, false, QB, PB, false>), g, dim3(kThreads), 0, s, b,
                           tiles_p, tiles_q);
    return hipGetLastError();
}

template <typename T, bool Q_RS, bool P_RS, int EPI>
hipError_t run(GemmOp op, const GemmArgs &a, hipStream_t s) {
    // the forward (both operands reduction-contiguous) may take 320 x 192,
    // the gradient (both reduction-strided) 192 x 320
    if constexpr ((EPI == EPI_LP || EPI == EPI_F32) && !Q_RS && !P_RS) {
        if (shape_for(op, a.rows, a.cols) == SHAPE_10x6) return run_shape<T, Q_RS, P_RS, EPI, 10, 6>(a, s);
    }
    if constexpr ((EPI == EPI_LP || EPI == EPI_F32) && Q_RS && P_RS) {
        if (shape_for(op, a.rows, a.cols) == SHAPE_6x10) return run_shape<T, Q_RS, P_RS, EPI, 6, 10>(a, s);
    }
    return run_shape<T, Q_RS, P_RS, EPI, 8, 8>(a, s);
}

template <typename T>
hipError_t dispatch(GemmOp op, const GemmArgs &a, hipStream_t s) {
    switch (op) {
        case GemmOp::Fwd:
            return a.out_f32 ? run<T, false, false, EPI_F32>(op, a, s) : run<T, false, false, EPI_LP>(op, a, s);
        case GemmOp::FwdGelu:
            return a.out_f32 ? run<T, false, false, EPI_GELU_F32A>(op, a, s) : run<T, false, false, EPI_GELU>(op, a, s);
        case GemmOp::Dx:
            return run<T, true, false, EPI_ACC>(op, a, s);
        case GemmOp::Dw:
            return a.out_f32 ? run<T, true, true, EPI_F32>(op, a, s) : run<T, true, true, EPI_LP>(op, a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

void gemm_tile(GemmOp op, int64_t rows, int64_t cols, int *tile_rows, int *tile_cols) {
    const Shape sh = (op == GemmOp::Fwd || op == GemmOp::Dw) ? shape_for(op, rows, cols) : SHAPE_8x8;
    *tile_cols = sh == SHAPE_10x6 ? 320 : (sh == SHAPE_6x10 ? 192 : 256);
    *tile_rows = sh == SHAPE_10x6 ? 192 : (sh == SHAPE_6x10 ? 320 : 256);
}

int64_t gemm_workgroups(GemmOp op, int64_t rows, int64_t cols) {
    int tp = 256, tq = 256;
    gemm_tile(op, rows, cols, &tp, &tq);
    return ((rows + tp - 1) / tp) * ((cols + tq - 1) / tq);
}

hipError_t launch_gemm(GemmOp op, int dtype, const GemmArgs &a, hipStream_t stream) {
    if (dtype == 1) return dispatch<_Float16>(op, a, stream);
    if (dtype == 2) return dispatch<__bf16>(op, a, stream);
    return hipErrorInvalidValue;
}

hipError_t build_gelu_tables(hipStream_t stream) {
    hipLaunchKernelGGL(gelu_table_kernel<_Float16>, dim3(256), dim3(256), 0, stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gelu_table_kernel<__bf16>, dim3(256), dim3(256), 0, stream);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(gelu_grad_table_kernel<_Float16>, dim3(256), dim3(256), 0, stream);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(gelu_grad_table_kernel<__bf16>, dim3(256), dim3(256), 0, stream);
    return hipGetLastError();
}

hipError_t launch_gelu_bwd(int dtype, const float *dH, const void *A, void *dA, int64_t count,
                           bool out_f32, hipStream_t stream) {
    if (count <= 0) return hipSuccess;
    // one workgroup of 1024 threads per compute unit (each holds the LDS
    // table), fewer for small counts
    const int64_t threads = (count + 7) / 8;
    int64_t blocks = (threads + 1023) / 1024;
    if (blocks > 256) blocks = 256;
    const uint16_t *a16 = static_cast<const uint16_t *>(A);
    const dim3 g((unsigned)blocks), b(1024);
    if (dtype == 1 && !out_f32)
        hipLaunchKernelGGL((gelu_bwd_kernel<_Float16, false>), g, b, 0, stream, dH, a16, dA, count);
    else if (dtype == 1)
        hipLaunchKernelGGL((gelu_bwd_kernel<_Float16, true>), g, b, 0, stream, dH, a16, dA, count);
    else if (dtype == 2 && !out_f32)
        hipLaunchKernelGGL((gelu_bwd_kernel<__bf16, false>), g, b, 0, stream, dH, a16, dA, count);
    else if (dtype == 2)
        hipLaunchKernelGGL((gelu_bwd_kernel<__bf16, true>), g, b, 0, stream, dH, a16, dA, count);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace zi
