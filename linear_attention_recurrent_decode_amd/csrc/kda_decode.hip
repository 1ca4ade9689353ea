// kda_decode.hip -- the kernel layer of libkda.so: the gfx950 kernels and
// their launches, reached from the host layer (kda_host.cpp: the C ABI of
// kda.h, argument validation, the launch plan) through kda_launch.h.
//
// Recurrent KDA decode is a bandwidth-bound stream over the state pool: per
// (request, value head) and call, a 64 KiB fp32 state tile is read once and
// written once, while the arithmetic per token is a few fused multiply-adds
// per state element.  Nothing here is a dense contraction, so nothing runs on
// the matrix cores; the design goals are every byte of the tile in flight at
// once, 16-byte coalesced accesses, and a short dependency chain per token.
//
// Work decomposition.  One wave64 owns 32 value columns x all 128 key rows of
// one (request, value head) tile: 4096 floats, 64 per lane, held in VGPRs for
// every token of the call.  Lane l holds columns 4*(l%8) .. +3 (one 16-byte
// vector per row) of the 16 key rows 16*(l/8) .. +15, so eight consecutive
// lanes read one row's 128 contiguous bytes.  Each of the 16 loads of a wave
// covers 8 rows x 128 bytes.  A workgroup is 1, 2 or 4 waves
// (a value tile of 32, 64 or 128 columns); the grid is one workgroup per
// (request, value head, value tile).  Columns never interact in the
// recurrence, so the tiling cannot change a single result bit: every wave runs
// the same per-column arithmetic in the same order whatever the tile width.
// Calls with several tokens per request or few tiles take two more layouts
// of the same arithmetic, with the same result bits: 16-column waves, one
// column of 32 key rows per lane (kda_decode_q_kernel), and split-key
// 16-column waves, one column of 16 key rows per lane, two waves per column
// set (kda_decode_split_kernel).
//
// Per token (vLLM PR 57585 names the op; the gated delta rule of Kimi Delta
// Attention is the recurrence):
//   a_i = exp(g_i)
//   u_j = sum_i S_ij (a_i k_i)      -- the correction against the decayed state
//   w_j = sum_i S_ij (a_i q_i)
//   kq  = sum_i k_i q_i
//   v'_j = beta (v_j - u_j)
//   o_j = scale (w_j + v'_j kq)     -- equals scale * sum_i S'_ij q_i
//   S'_ij = a_i S_ij + k_i v'_j
// so both key-axis reductions come from one pass over the old state, and the
// only cross-lane step per token is one 3-level reduction (DPP and permlane
// swaps, no LDS) over the 8 lanes that share a column group.  The gated
// RMSNorm epilogue (b12x PR 249, walkthrough: normalise and gate the decoded
// output) needs the sum of o^2 over all 128 columns, which forces the 4-wave
// tile and adds one LDS exchange per token.
//
// Options of the same kernels: a bf16 state pool (widened exactly on load,
// rounded once on write-back), the gate activation fused from raw
// projections (FlashInfer PR 4562's binding passes raw_gate, raw_beta, A_log
// and dt_bias), the state after every token for speculative decoding, and a
// one-workgroup metadata check that makes a call all or nothing.

#include <hip/hip_runtime.h>

#include <atomic>
#include <stdint.h>
#include <string.h>
#include <type_traits>
#include <utility>

#include "kda_launch.h"

namespace {

constexpr int KD = 128;           // key head size handled by the kernels
constexpr int VD = 128;           // value head size handled by the kernels
constexpr int ROWS_PER_LANE = 16;  // 128 key rows over 8 row groups
constexpr int MAX_DEVICES = 64;

// Field order matters: what a workgroup needs before its first token's loads
// (the token inputs and their strides) comes first, so that it arrives in
// one batch of scalar loads from the kernel arguments.
struct DecodeParams {
    const uint16_t *q;
    const uint16_t *k;
    const uint16_t *v;
    const float *g;
    const float *beta;
    const uint16_t *raw_gate;    // fused gate activation (template parameter RAWG)
    const uint16_t *raw_beta;
    const float *A_log;
    const float *dt_bias;
    int64_t q_stride, k_stride, v_stride, g_stride, beta_stride, raw_gate_stride, raw_beta_stride;
    int32_t HV, T;
    uint32_t qk_magic, qk_magic_hi;   // q/k head of value head hv: qk_head(hv)
    float scale, eps;
    void *state;                 // fp32 or bf16 pool (template parameter BF16S)
    const int32_t *slot_idx;
    const int32_t *cu_seqlens;   // NULL: fixed T tokens per request
    uint16_t *out;
    const uint16_t *gate;
    const uint16_t *norm_weight;
    int64_t out_stride, gate_stride;
    int64_t num_slots, slot_stride;
    int32_t *status;             // KDA_FLAG_VALIDATE: the metadata check's verdict
    void *inter_state;           // NULL, or the state after every token (pool element type)
    int64_t inter_stride;
    int64_t tokens;              // host side: token rows of the call
    int32_t check_in_kernel;     // host side: launch the instances that check the metadata (VCHECK)
};

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two fp32 -> packed bf16 (lo in bits 0..15), round to nearest even, in one
// gfx950 v_cvt_pk_bf16_f32.  Checked on the device against the integer
// rounding (add 0x7FFF plus the lowest kept bit, drop 16 bits) over all 2^32
// fp32 bit patterns: identical for every non-NaN input, denormals and ties
// included; a NaN stays a NaN.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    const f32x2 x = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}

__device__ __forceinline__ float silu(float z)
{
    return z / (1.0f + __expf(-z));
}

// Fused gate activation (FlashInfer PR 4562, inline review of the binding:
// the kernel takes raw_gate, raw_beta, A_log and dt_bias; the activation is
// the gate of Kimi Delta Attention):
//   g = -A softplus(raw + bias),  A = exp(A_log),  beta = sigmoid(raw_beta).
// softplus is taken as max(x, 0) + log(1 + e^-|x|), which cannot overflow:
// +inf gives g = -inf (the key row is cleared), -inf gives g = 0.  Both
// transcendentals are the hardware's base-2 exp and log (one instruction
// each; the log's argument 1 + e^-|x| lies in [1, 2], where v_log_f32 needs
// no range handling).  The only loss against log1p is the rounding of
// 1 + e^-|x|, at most 2^-24 absolute in softplus, so |dg| <= 2^-24 A plus a
// few ulp of g: a relative change of the decay factor far below the fp32
// state rounding of a call.  (The device library's log1pf expands to over a
// hundred instructions, f64 steps included.)  Every body evaluates these two
// functions on the same fp32 operands, so they agree bit for bit wherever
// the activation happens.
__device__ __forceinline__ float gate_log_decay(float raw, float bias, float A)
{
    constexpr float LN2 = 0.693147180559945309f;
    const float x = raw + bias;
    const float sp = fmaxf(x, 0.0f) + LN2 * __builtin_amdgcn_logf(1.0f + __expf(-fabsf(x)));
    return -A * sp;
}

__device__ __forceinline__ float beta_from_raw(float r)
{
    return 1.0f / (1.0f + __expf(-r));
}

// The lane's 16 rows x 4 columns of a state tile in HBM.  fp32 state moves as
// one 16-byte vector per row; bf16 state (BF16S) as one 8-byte vector per row,
// widened exactly to fp32 on load and rounded to nearest even on store.  The
// math in between is fp32 in both cases.  Both directions are non-temporal:
// the tile is read once and written once per call.
template <bool BF16S>
struct TileIO {
    using chunk = typename std::conditional<BF16S, u32x2, f32x4>::type;
    chunk *ptr;

    __device__ __forceinline__ TileIO(void *state, int64_t elem_offset)
        : ptr(reinterpret_cast<chunk *>(static_cast<char *>(state) + elem_offset * (BF16S ? 2 : 4))) {}

    __device__ __forceinline__ f32x4 load(int row) const
    {
        if constexpr (BF16S) {
            const u32x2 r = __builtin_nontemporal_load(ptr + row * (VD / 4));
            return f32x4{bf16_lo(r.x), bf16_hi(r.x), bf16_lo(r.y), bf16_hi(r.y)};
        } else {
            return __builtin_nontemporal_load(ptr + row * (VD / 4));
        }
    }

    __device__ __forceinline__ void store(int row, f32x4 v) const
    {
        if constexpr (BF16S) {
            const u32x2 r = {pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)};
            __builtin_nontemporal_store(r, ptr + row * (VD / 4));
        } else {
            __builtin_nontemporal_store(v, ptr + row * (VD / 4));
        }
    }
};

// DPP lane moves (gfx9 DPP controls).
#define KDA_DPP(x, ctrl)                                                                                   \
    __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, (x)), (ctrl), 0xF, 0xF, \
                                                          false))
constexpr int DPP_ROW_ROR8 = 0x128;          // lane l <- l^8 within its 16-lane row
constexpr int DPP_ROW_HALF_MIRROR = 0x141;   // lane l <- 7 - l within its 8-lane half row
constexpr int DPP_ROW_MIRROR = 0x140;        // lane l <- 15 - l within its 16-lane row
constexpr int DPP_ROW_SR1 = 0x111;           // lane l <- l - 1 within its 16-lane row
constexpr int DPP_QUAD_XOR1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;          // quad_perm [2,3,0,1]

// gfx950 v_permlane16_swap / v_permlane32_swap exchange the odd 16-lane rows
// (upper 32 lanes) of `a` with the even rows (lower 32 lanes) of `b`; with
// a = b = x, a + b then pairs every lane with lane l^16 (l^32).  Both
// registers are read and written, so they are in-out operands; the s_nop
// pads give the two wait states a VALU result needs before these read it
// (and before a DPP reads theirs).
__device__ __forceinline__ float add_permlane16_swap(float x)
{
    uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
    return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

__device__ __forceinline__ float add_permlane32_swap(float x)
{
    uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
    return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

// Three values at once over lane pairs l, l^16 and then l, l^32 (the
// quarters of a 16-column wave): the same additions as add_permlane16_swap
// and add_permlane32_swap on each value, with the three swaps of a level
// issued back to back between one pair of wait-state pads.
__device__ __forceinline__ void add_swaps3(float &x, float &y, float &z)
{
    uint32_t x0 = __builtin_bit_cast(uint32_t, x), x1 = x0;
    uint32_t y0 = __builtin_bit_cast(uint32_t, y), y1 = y0;
    uint32_t z0 = __builtin_bit_cast(uint32_t, z), z1 = z0;
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\tv_permlane16_swap_b32 %2, %3\n\t"
                 "v_permlane16_swap_b32 %4, %5\n\ts_nop 1"
                 : "+v"(x0), "+v"(x1), "+v"(y0), "+v"(y1), "+v"(z0), "+v"(z1));
    x = __builtin_bit_cast(float, x0) + __builtin_bit_cast(float, x1);
    y = __builtin_bit_cast(float, y0) + __builtin_bit_cast(float, y1);
    z = __builtin_bit_cast(float, z0) + __builtin_bit_cast(float, z1);
    x0 = x1 = __builtin_bit_cast(uint32_t, x);
    y0 = y1 = __builtin_bit_cast(uint32_t, y);
    z0 = z1 = __builtin_bit_cast(uint32_t, z);
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\tv_permlane32_swap_b32 %2, %3\n\t"
                 "v_permlane32_swap_b32 %4, %5\n\ts_nop 1"
                 : "+v"(x0), "+v"(x1), "+v"(y0), "+v"(y1), "+v"(z0), "+v"(z1));
    x = __builtin_bit_cast(float, x0) + __builtin_bit_cast(float, x1);
    y = __builtin_bit_cast(float, y0) + __builtin_bit_cast(float, y1);
    z = __builtin_bit_cast(float, z0) + __builtin_bit_cast(float, z1);
}

// The same two levels for the split-key waves, which need the three sums
// only in LDS: u and w share their first swap, k.q joins them in the second,
// and the sums end spread over the rows, u in row 0, w in row 1, k.q in rows
// 2 and 3 (each addition has the operands, in the same order, that
// add_swaps3 gives it, so the bits are the same; 8 VALU instructions in
// place of 18).
__device__ __forceinline__ float spread_swaps3(float u, float w, float kq)
{
    uint32_t a = __builtin_bit_cast(uint32_t, u), b = __builtin_bit_cast(uint32_t, w);
    uint32_t k0 = __builtin_bit_cast(uint32_t, kq), k1 = k0;
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\tv_permlane16_swap_b32 %2, %3\n\ts_nop 1"
                 : "+v"(a), "+v"(b), "+v"(k0), "+v"(k1));
    // a = rows (u0, w0, u2, w2), b = (u1, w1, u3, w3): the pair sums of u in
    // rows 0 and 2, of w in rows 1 and 3
    uint32_t c = __builtin_bit_cast(uint32_t, __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b));
    uint32_t d = __builtin_bit_cast(uint32_t, __builtin_bit_cast(float, k0) + __builtin_bit_cast(float, k1));
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(c), "+v"(d));
    // c = rows (u01, w01, kq01, kq01), d = (u23, w23, kq23, kq23)
    return __builtin_bit_cast(float, c) + __builtin_bit_cast(float, d);
}

// Sum over the 8 lanes that share a column group (lane bits 3..5: lanes l,
// l+8, .., l+56), all on the VALU.  Each level adds the same two operands on
// both lanes of a pair, so every lane of the group ends with the same bits,
// and the order of additions is the same for every tile width.
__device__ __forceinline__ float sum_row_groups(float x)
{
    x += KDA_DPP(x, DPP_ROW_ROR8);
    x = add_permlane16_swap(x);
    return add_permlane32_swap(x);
}

// Four values' sums over the row groups at once, for the 32-column waves:
// the l^8 level as in sum_row_groups, then the two swap levels shared by the
// four values, which end spread over the 16-lane rows (row r holds the sum
// of x_r; each addition has the operands, in the same order, that
// sum_row_groups gives it, so the bits are the same).
__device__ __forceinline__ float spread_row_groups4(float x0, float x1, float x2, float x3)
{
    x0 += KDA_DPP(x0, DPP_ROW_ROR8);
    x1 += KDA_DPP(x1, DPP_ROW_ROR8);
    x2 += KDA_DPP(x2, DPP_ROW_ROR8);
    x3 += KDA_DPP(x3, DPP_ROW_ROR8);
    uint32_t a = __builtin_bit_cast(uint32_t, x0), b = __builtin_bit_cast(uint32_t, x1);
    uint32_t c = __builtin_bit_cast(uint32_t, x2), d = __builtin_bit_cast(uint32_t, x3);
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\tv_permlane16_swap_b32 %2, %3\n\ts_nop 1"
                 : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
    // a = rows (x0 of row 0, x1 of row 0, x0 of row 2, x1 of row 2), b the
    // same of rows 1 and 3; c, d for x2, x3
    uint32_t e = __builtin_bit_cast(uint32_t, __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b));
    uint32_t f = __builtin_bit_cast(uint32_t, __builtin_bit_cast(float, c) + __builtin_bit_cast(float, d));
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(e), "+v"(f));
    // e = rows (x0, x1, x2, x3 over rows 0 + 1), f the same over rows 2 + 3
    return __builtin_bit_cast(float, e) + __builtin_bit_cast(float, f);
}

// The four row values of a spread sum (row r holds x_r) in every lane.
__device__ __forceinline__ void gather_rows4(float x, float &x0, float &x1, float &x2, float &x3)
{
    uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
    // a = rows (x0, x0, x2, x2), b = (x1, x1, x3, x3)
    uint32_t a2 = a, b2 = b;   // copies made by VALU moves: the leading s_nop covers them
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\tv_permlane32_swap_b32 %2, %3\n\ts_nop 1"
                 : "+v"(a), "+v"(a2), "+v"(b), "+v"(b2));
    x0 = __builtin_bit_cast(float, a);
    x2 = __builtin_bit_cast(float, a2);
    x1 = __builtin_bit_cast(float, b);
    x3 = __builtin_bit_cast(float, b2);
}

// Sum over the 8 column groups of a wave (lane bits 0..2): pairs l <-> 7-l,
// then l <-> l^1, then l <-> l^2, all symmetric, all on the VALU.
__device__ __forceinline__ float sum_col_groups(float x)
{
    x += KDA_DPP(x, DPP_ROW_HALF_MIRROR);
    x += KDA_DPP(x, DPP_QUAD_XOR1);
    x += KDA_DPP(x, DPP_QUAD_XOR2);
    return x;
}

// One token's inputs as a lane needs them: q, k over its 16 key rows, v over
// its 4 value columns, beta of the head, and g of only 2 of its 16 key rows
// (rows row0 + 2 cg and + 1, cg = the lane's column group): each lane takes
// the exponential of its 2 rows and the 8 lanes of the row group exchange
// the decay factors (bcast8), instead of all 8 computing all 16.  With the
// fused gate activation (RAWG) g.x carries the 2 rows' raw bf16 values, which
// the lane activates first, and beta the raw beta's bits (zero-extended by
// the load; widened where it is used, so that nothing waits for the load
// before the state tile's loads are issued).
struct TokenIn {
    uint4 k0, k1, q0, q1;
    float2 g;
    uint2 v;
    float beta;
};

// What the fused gate activation needs besides the token: A_log of the head
// and dt_bias of the lane's 2 key rows, loaded once per call.  A = exp(A_log)
// is evaluated where it is used, so that no load of the state tile waits for
// A_log to arrive.
template <bool RAWG>
struct HeadGate {
    __device__ __forceinline__ void load(const DecodeParams &, int, int, int) {}
};

template <>
struct HeadGate<true> {
    float2 b;
    float a_log;
    __device__ __forceinline__ void load(const DecodeParams &p, int hv, int row0, int cg)
    {
        b = reinterpret_cast<const float2 *>(p.dt_bias + (int64_t)hv * KD + row0)[cg];
        a_log = p.A_log[hv];
    }
};

// x of lane 8 (lane / 8) + I: a broadcast within each group of 8 lanes, on
// the VALU (no LDS-pipe round trip to wait for).  A quad_perm broadcast of
// lane I % 4 serves the quad that holds lane I; the other quad of the group
// takes it with a 4-lane row shift whose bank mask writes only that quad
// (banks are the 4-lane quarters of a 16-lane row).
template <int I>
__device__ __forceinline__ float bcast8(float x)
{
    static_assert(I >= 0 && I < 8, "lane within a group of 8");
    constexpr int DPP_ROW_SHL4 = 0x104;   // lane l <- l + 4 within its row
    constexpr int DPP_ROW_SHR4 = 0x114;   // lane l <- l - 4 within its row
    const int q = __builtin_amdgcn_update_dpp(0, __float_as_int(x), (I & 3) * 0x55, 0xF, 0xF, false);
    const int r = I < 4 ? __builtin_amdgcn_update_dpp(q, q, DPP_ROW_SHR4, 0xF, 0xA, false)   // upper quads
                        : __builtin_amdgcn_update_dpp(q, q, DPP_ROW_SHL4, 0xF, 0x5, false);  // lower quads
    return __int_as_float(r);
}

template <bool RAWG>
__device__ __forceinline__ void load_token(TokenIn &in, const DecodeParams &p, int64_t t, int h, int hv, int row0,
                                           int col)
{
    const uint4 *kp = reinterpret_cast<const uint4 *>(p.k + t * p.k_stride + h * KD + row0);
    const uint4 *qp = reinterpret_cast<const uint4 *>(p.q + t * p.q_stride + h * KD + row0);
    in.k0 = kp[0];
    in.k1 = kp[1];
    in.q0 = qp[0];
    in.q1 = qp[1];
    const int cg = (col >> 2) & 7;
    if constexpr (RAWG) {
        const uint32_t *rp = reinterpret_cast<const uint32_t *>(p.raw_gate + t * p.raw_gate_stride + (int64_t)hv * KD + row0);
        in.g.x = __uint_as_float(rp[cg]);
        in.beta = __uint_as_float((uint32_t)p.raw_beta[t * p.raw_beta_stride + hv]);
    } else {
        in.g = reinterpret_cast<const float2 *>(p.g + t * p.g_stride + (int64_t)hv * KD + row0)[cg];
        in.beta = p.beta[t * p.beta_stride + hv];
    }
    in.v = *reinterpret_cast<const uint2 *>(p.v + t * p.v_stride + (int64_t)hv * VD + col);
}

// Advance the lane's part of the state by one token and write its output.
// Every floating-point operation is spelled out (explicit fmaf, no implicit
// contraction), so each inlined copy of this function rounds identically.
// With PREFETCH the next token's inputs are loaded into `in` as soon as this
// token's are unpacked, so they are in flight while this token computes.
// SPREAD: the key-axis sums over the row groups by the shared swaps of
// spread_row_groups4 (u then gathered into every lane, w left spread, so that
// without the norm each 16-lane row forms one column's output): 25 fewer VALU
// instructions per token, the same bits.  Measured on MI355X it pays on the
// tokens after a request's first (N80/T4 17.59 vs 18.43 us, N96/T4 19.83 vs
// 20.06, N72/T2 14.78 vs 14.92; N90/T3 17.25 vs 17.10 the other way) but
// not on a one-token call (N24/T1 5.42 vs 5.38), so the first token keeps
// the replicated sums.
template <bool NORM, bool PREFETCH, bool RAWG, bool SPREAD = false>
__device__ __forceinline__ void advance_token(f32x4 (&s)[ROWS_PER_LANE], TokenIn &in, const DecodeParams &p,
                                              const HeadGate<RAWG> &hg, int64_t t, int64_t eos, int h, int hv,
                                              int lane, int wave, int rg, int row0, int col,
                                              float (&norm_partial)[2][4])
{
    // unpack; the decay factors a_i = exp(g_i): this lane's 2 rows, then all
    // 16 rows of the row group from its 8 lanes
    float kk[ROWS_PER_LANE], qq[ROWS_PER_LANE], a[ROWS_PER_LANE];
    const uint32_t kw[8] = {in.k0.x, in.k0.y, in.k0.z, in.k0.w, in.k1.x, in.k1.y, in.k1.z, in.k1.w};
    const uint32_t qw[8] = {in.q0.x, in.q0.y, in.q0.z, in.q0.w, in.q1.x, in.q1.y, in.q1.z, in.q1.w};
    float b, g_lo, g_hi;
    if constexpr (RAWG) {
        const uint32_t rw = __float_as_uint(in.g.x);
        const float A = expf(hg.a_log);
        g_lo = gate_log_decay(bf16_lo(rw), hg.b.x, A);
        g_hi = gate_log_decay(bf16_hi(rw), hg.b.y, A);
        b = beta_from_raw(bf16_lo(__float_as_uint(in.beta)));
    } else {
        g_lo = in.g.x;
        g_hi = in.g.y;
        b = in.beta;
    }
    const float a_lo = __expf(g_lo), a_hi = __expf(g_hi);
    a[0] = bcast8<0>(a_lo), a[1] = bcast8<0>(a_hi);
    a[2] = bcast8<1>(a_lo), a[3] = bcast8<1>(a_hi);
    a[4] = bcast8<2>(a_lo), a[5] = bcast8<2>(a_hi);
    a[6] = bcast8<3>(a_lo), a[7] = bcast8<3>(a_hi);
    a[8] = bcast8<4>(a_lo), a[9] = bcast8<4>(a_hi);
    a[10] = bcast8<5>(a_lo), a[11] = bcast8<5>(a_hi);
    a[12] = bcast8<6>(a_lo), a[13] = bcast8<6>(a_hi);
    a[14] = bcast8<7>(a_lo), a[15] = bcast8<7>(a_hi);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        kk[2 * i] = bf16_lo(kw[i]);
        kk[2 * i + 1] = bf16_hi(kw[i]);
        qq[2 * i] = bf16_lo(qw[i]);
        qq[2 * i + 1] = bf16_hi(qw[i]);
    }
    // k.q over the lane's 16 rows as a pairwise tree (row pairs 2m, 2m + 1,
    // then pairs of pairs): the order in which the 16-column-wave kernel,
    // whose lanes own one row pair each, adds them across lanes
    float kp[ROWS_PER_LANE / 2];
#pragma unroll
    for (int m = 0; m < ROWS_PER_LANE / 2; ++m)
        kp[m] = fmaf(kk[2 * m + 1], qq[2 * m + 1], kk[2 * m] * qq[2 * m]);
    float kq = ((kp[0] + kp[1]) + (kp[2] + kp[3])) + ((kp[4] + kp[5]) + (kp[6] + kp[7]));
    const float v0 = bf16_lo(in.v.x), v1 = bf16_hi(in.v.x), v2 = bf16_lo(in.v.y), v3 = bf16_hi(in.v.y);
    if constexpr (PREFETCH) {
        if (t + 1 < eos)
            load_token<RAWG>(in, p, t + 1, h, hv, row0, col);
    }

    // one pass over the old state: both key-axis partial sums, each chain
    // opened by its first row's products
    float u0, u1, u2, u3, w0, w1, w2, w3;
    {
        const float ak = a[0] * kk[0], aq = a[0] * qq[0];
        u0 = s[0].x * ak;
        u1 = s[0].y * ak;
        u2 = s[0].z * ak;
        u3 = s[0].w * ak;
        w0 = s[0].x * aq;
        w1 = s[0].y * aq;
        w2 = s[0].z * aq;
        w3 = s[0].w * aq;
    }
#pragma unroll
    for (int i = 1; i < ROWS_PER_LANE; ++i) {
        const float ak = a[i] * kk[i], aq = a[i] * qq[i];
        u0 = fmaf(s[i].x, ak, u0);
        u1 = fmaf(s[i].y, ak, u1);
        u2 = fmaf(s[i].z, ak, u2);
        u3 = fmaf(s[i].w, ak, u3);
        w0 = fmaf(s[i].x, aq, w0);
        w1 = fmaf(s[i].y, aq, w1);
        w2 = fmaf(s[i].z, aq, w2);
        w3 = fmaf(s[i].w, aq, w3);
    }
    kq = sum_row_groups(kq);
    // u in every lane (the update needs all four columns' v'); with SPREAD
    // and without the norm w only where o is formed: each 16-lane row r
    // forms o of column 4 cg + r
    constexpr bool SPREAD_W = SPREAD && !NORM;
    if constexpr (SPREAD) {
        gather_rows4(spread_row_groups4(u0, u1, u2, u3), u0, u1, u2, u3);
    } else {
        u0 = sum_row_groups(u0);
        u1 = sum_row_groups(u1);
        u2 = sum_row_groups(u2);
        u3 = sum_row_groups(u3);
    }
    float w_row = 0.f;
    if constexpr (SPREAD_W) {
        w_row = spread_row_groups4(w0, w1, w2, w3);
    } else {
        w0 = sum_row_groups(w0);
        w1 = sum_row_groups(w1);
        w2 = sum_row_groups(w2);
        w3 = sum_row_groups(w3);
    }

    // delta correction, readout, rank-1 update
    const float vp0 = b * (v0 - u0);
    const float vp1 = b * (v1 - u1);
    const float vp2 = b * (v2 - u2);
    const float vp3 = b * (v3 - u3);
    float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f, o_row = 0.f;
    if constexpr (!SPREAD_W) {
        o0 = p.scale * fmaf(vp0, kq, w0);
        o1 = p.scale * fmaf(vp1, kq, w1);
        o2 = p.scale * fmaf(vp2, kq, w2);
        o3 = p.scale * fmaf(vp3, kq, w3);
    } else {
        const int r = lane >> 4;
        const float vp_row = r == 0 ? vp0 : r == 1 ? vp1 : r == 2 ? vp2 : vp3;
        o_row = p.scale * fmaf(vp_row, kq, w_row);
    }
#pragma unroll
    for (int i = 0; i < ROWS_PER_LANE; ++i) {
        s[i].x = fmaf(kk[i], vp0, a[i] * s[i].x);
        s[i].y = fmaf(kk[i], vp1, a[i] * s[i].y);
        s[i].z = fmaf(kk[i], vp2, a[i] * s[i].z);
        s[i].w = fmaf(kk[i], vp3, a[i] * s[i].w);
    }

    if constexpr (NORM) {
        // gated RMSNorm over the head's 128 columns: the four waves of the
        // workgroup hold 32 columns each and meet in LDS.  The gate and
        // weight are loaded here, off the state tile's critical path.
        const uint2 zz = *reinterpret_cast<const uint2 *>(p.gate + t * p.gate_stride + (int64_t)hv * VD + col);
        const uint2 nw = *reinterpret_cast<const uint2 *>(p.norm_weight + col);
        float ss = fmaf(o3, o3, fmaf(o2, o2, fmaf(o1, o1, o0 * o0)));
        ss = sum_col_groups(ss);
        float *slot_sum = norm_partial[t & 1];
        if (lane == 0)
            slot_sum[wave] = ss;
        __syncthreads();
        const float total = (slot_sum[0] + slot_sum[1]) + (slot_sum[2] + slot_sum[3]);
        const float r = rsqrtf(fmaf(total, 1.0f / VD, p.eps));
        o0 = o0 * r * bf16_lo(nw.x) * silu(bf16_lo(zz.x));
        o1 = o1 * r * bf16_hi(nw.x) * silu(bf16_hi(zz.x));
        o2 = o2 * r * bf16_lo(nw.y) * silu(bf16_lo(zz.y));
        o3 = o3 * r * bf16_hi(nw.y) * silu(bf16_hi(zz.y));
    }
    if constexpr (!SPREAD_W) {
        if (rg == 0) {
            uint2 packed;
            packed.x = pack_bf16x2(o0, o1);
            packed.y = pack_bf16x2(o2, o3);
            *reinterpret_cast<uint2 *>(p.out + t * p.out_stride + (int64_t)hv * VD + col) = packed;
        }
    } else {
        // lanes 16 r + cg (row group 2 r) store column 4 cg + r
        if ((lane & 8) == 0)
            p.out[t * p.out_stride + (int64_t)hv * VD + col + (lane >> 4)] = (uint16_t)pack_bf16x2(o_row, 0.0f);
    }
}

// Token inputs of up to STAGE_TOKENS tokens of one (request, value head),
// staged in LDS by the whole workgroup: q, k, g over all 128 key rows, v over
// the workgroup's columns, beta.
constexpr int STAGE_TOKENS = 4;

// Tokens of the next chunk to stage: min(remaining, STAGE_TOKENS), in integers
// (the device library's 64-bit min goes through doubles).
__device__ __forceinline__ int chunk_tokens(int64_t remaining)
{
    return remaining < STAGE_TOKENS ? (int)remaining : STAGE_TOKENS;
}

template <int NW>
struct TokenStage {
    uint4 k[STAGE_TOKENS][KD / 8];
    uint4 q[STAGE_TOKENS][KD / 8];
    float4 g[STAGE_TOKENS][KD / 4];
    uint2 v[STAGE_TOKENS][NW * 8];
    float beta[STAGE_TOKENS];
};

// Cooperative global -> LDS copy of tokens t0 .. t0+nt-1 (nt <= STAGE_TOKENS),
// in two halves so that the state tile's loads can be issued in between: the
// loads into registers, then (after the tile's loads) the LDS writes.  With
// the fused gate activation (RAWG) the raw gate arrives as bf16 pieces of 8
// key channels with their 8 dt_bias values, and the activation runs once per
// channel in stage_store, so LDS holds the activated g and beta either way.
template <int NW, bool RAWG>
struct StagePieces {
    static constexpr int THREADS = 64 * NW;
    static constexpr int G_PIECES = RAWG ? KD / 8 : KD / 4;      // 16-byte pieces of g (or raw gate)
    static constexpr int PIECES = KD / 8 + KD / 8 + G_PIECES;    // ... of k, q and g per token
    static constexpr int ITER = (STAGE_TOKENS * PIECES + THREADS - 1) / THREADS;
    static constexpr int VITER = (STAGE_TOKENS * NW * 8 + THREADS - 1) / THREADS;
    uint4 kqg[ITER];
    float4 bias[RAWG ? ITER : 1][2];
    uint2 v[VITER];
    float beta;
};

template <int NW, bool RAWG>
__device__ __forceinline__ void stage_load(StagePieces<NW, RAWG> &r, const DecodeParams &p, int64_t t0, int nt,
                                           int h, int hv, int col0)
{
    using SP = StagePieces<NW, RAWG>;
    const int tid = threadIdx.x;
#pragma unroll
    for (int it = 0; it < SP::ITER; ++it) {
        const int idx = tid + it * SP::THREADS;
        if (idx < nt * SP::PIECES) {
            const int j = idx / SP::PIECES, e = idx - j * SP::PIECES;
            const int64_t t = t0 + j;
            // one load per piece from a selected address (no divergent branches,
            // whose loads into one register would have to wait for each other)
            const uint4 *gsrc =
                RAWG ? reinterpret_cast<const uint4 *>(p.raw_gate + t * p.raw_gate_stride + (int64_t)hv * KD)
                     : reinterpret_cast<const uint4 *>(p.g + t * p.g_stride + (int64_t)hv * KD);
            const uint4 *src = e < KD / 8   ? reinterpret_cast<const uint4 *>(p.k + t * p.k_stride + h * KD) + e
                               : e < KD / 4 ? reinterpret_cast<const uint4 *>(p.q + t * p.q_stride + h * KD) + (e - KD / 8)
                                            : gsrc + (e - KD / 4);
            r.kqg[it] = *src;
            if constexpr (RAWG) {
                // dt_bias of the piece's 8 key channels (k and q pieces read
                // channels 0..7 and ignore them)
                const int m = e < KD / 4 ? 0 : e - KD / 4;
                const float4 *bp = reinterpret_cast<const float4 *>(p.dt_bias + (int64_t)hv * KD) + 2 * m;
                r.bias[it][0] = bp[0];
                r.bias[it][1] = bp[1];
            }
        }
    }
#pragma unroll
    for (int it = 0; it < SP::VITER; ++it) {
        const int idx = tid + it * SP::THREADS;
        if (idx < nt * NW * 8) {
            const int j = idx / (NW * 8), e = idx - j * (NW * 8);
            r.v[it] = reinterpret_cast<const uint2 *>(p.v + (t0 + j) * p.v_stride + (int64_t)hv * VD + col0)[e];
        }
    }
    if (tid < nt) {
        if constexpr (RAWG)   // the bits: widened in stage_store, after the tile's loads are issued
            r.beta = __uint_as_float((uint32_t)p.raw_beta[(t0 + tid) * p.raw_beta_stride + hv]);
        else
            r.beta = p.beta[(t0 + tid) * p.beta_stride + hv];
    }
}

template <int NW, bool RAWG>
__device__ __forceinline__ void stage_store(TokenStage<NW> &st, const StagePieces<NW, RAWG> &r, int nt, float A)
{
    using SP = StagePieces<NW, RAWG>;
    const int tid = threadIdx.x;
#pragma unroll
    for (int it = 0; it < SP::ITER; ++it) {
        const int idx = tid + it * SP::THREADS;
        if (idx < nt * SP::PIECES) {
            const int j = idx / SP::PIECES, e = idx - j * SP::PIECES;
            if (e < KD / 8) {
                st.k[j][e] = r.kqg[it];
            } else if (e < KD / 4) {
                st.q[j][e - KD / 8] = r.kqg[it];
            } else if constexpr (RAWG) {
                const int m = e - KD / 4;
                const uint4 w = r.kqg[it];
                const float4 b0 = r.bias[it][0], b1 = r.bias[it][1];
                st.g[j][2 * m] = float4{gate_log_decay(bf16_lo(w.x), b0.x, A), gate_log_decay(bf16_hi(w.x), b0.y, A),
                                        gate_log_decay(bf16_lo(w.y), b0.z, A), gate_log_decay(bf16_hi(w.y), b0.w, A)};
                st.g[j][2 * m + 1] =
                    float4{gate_log_decay(bf16_lo(w.z), b1.x, A), gate_log_decay(bf16_hi(w.z), b1.y, A),
                           gate_log_decay(bf16_lo(w.w), b1.z, A), gate_log_decay(bf16_hi(w.w), b1.w, A)};
            } else {
                st.g[j][e - KD / 4] = __builtin_bit_cast(float4, r.kqg[it]);
            }
        }
    }
#pragma unroll
    for (int it = 0; it < SP::VITER; ++it) {
        const int idx = tid + it * SP::THREADS;
        if (idx < nt * NW * 8) {
            const int j = idx / (NW * 8), e = idx - j * (NW * 8);
            st.v[j][e] = r.v[it];
        }
    }
    if (tid < nt)
        st.beta[tid] = RAWG ? beta_from_raw(bf16_lo(__float_as_uint(r.beta))) : r.beta;
}

__device__ __forceinline__ void read_staged(TokenIn &in, const uint4 (&k)[KD / 8], const uint4 (&q)[KD / 8],
                                            const float4 (&g)[KD / 4], uint2 v, float beta, int rg, int cg)
{
    in.k0 = k[2 * rg];
    in.k1 = k[2 * rg + 1];
    in.q0 = q[2 * rg];
    in.q1 = q[2 * rg + 1];
    in.g = reinterpret_cast<const float2 *>(g)[8 * rg + cg];   // key rows 16 rg + 2 cg, + 1
    in.v = v;
    in.beta = beta;
}

// hv / (HV / H), the q/k head that value head hv reads, as a multiply by
// m = floor(2^32 / d) + 1 (d = HV / H; m = m_lo + 2^32 m_hi): for n d < 2^32,
// floor(n m / 2^32) = floor(n / d) (the error term n (d - 2^32 mod d) / 2^32
// stays below 1 - (n mod d) / d).  The host checks HV < 65536, so n < HV and
// d <= HV keep n d < 2^32.  A scalar division would cost some thirty
// dependent instructions at the start of every workgroup.
__device__ __forceinline__ int qk_head(const DecodeParams &p, int hv)
{
    return (int)(__umulhi((uint32_t)hv, p.qk_magic) + (uint32_t)hv * p.qk_magic_hi);
}

// Three bodies of the 32-column kernel share advance_token and round
// identically (the launch plan sends many calls to the 16-column waves
// instead; these are the bodies of the calls it keeps here):
//   BODY_LOOP: the token loop prefetches token t+1 while token t computes;
//     the first token's inputs go out just before the state tile.  The
//     32-column body for one token per request from two tiles per compute
//     unit up with an fp32 pool.
//   BODY_PEELED: the first token is peeled off the loop and the tile's loads
//     are issued around the first token's input loads (4 rows, the inputs,
//     12 rows), pinned by scheduling fences; later tokens load at the top of
//     their iteration.  Fastest among the three for step calls with several
//     tokens per request, for launches below two tiles per compute unit
//     (the one-token serving shape), with the fused gate activation and with
//     a bf16 pool.
//   BODY_STAGED: the workgroup copies the inputs of up to STAGE_TOKENS tokens
//     into LDS while the tile is in flight, so the token loop reads no global
//     memory (longer requests restage in chunks; with a bf16 pool they load
//     the remaining tokens directly).  Fastest among the three for packed
//     batches of mixed lengths.
// The kernel arguments that a token's loads need, requested together with
// the slot index, so that the two scalar round trips overlap: the asm takes
// them all in SGPRs, so each of their loads is issued before it and one
// wait covers them.  Only for kernels that load a token's inputs before the
// state tile: otherwise the tile's loads go out first, right after the slot
// arrives, and these arguments follow (measured on MI355X: requesting them
// early delays the tile by about 0.3 us at one token and a few tiles).
template <bool RAWG>
__device__ __forceinline__ void slot_and_token_args(const DecodeParams &p, int64_t slot)
{
    if constexpr (RAWG)
        asm volatile("" ::"s"(slot), "s"(p.q), "s"(p.k), "s"(p.v), "s"(p.raw_gate), "s"(p.raw_beta), "s"(p.A_log),
                     "s"(p.dt_bias), "s"(p.q_stride), "s"(p.k_stride), "s"(p.v_stride), "s"(p.raw_gate_stride),
                     "s"(p.raw_beta_stride), "s"(p.qk_magic), "s"(p.qk_magic_hi));
    else
        asm volatile("" ::"s"(slot), "s"(p.q), "s"(p.k), "s"(p.v), "s"(p.g), "s"(p.beta), "s"(p.q_stride),
                     "s"(p.k_stride), "s"(p.v_stride), "s"(p.g_stride), "s"(p.beta_stride), "s"(p.qk_magic),
                     "s"(p.qk_magic_hi));
}

// The metadata check of a validated call of at most CHECK_IN_WAVE requests,
// done by every wave of the decode itself instead of a kernel of its own:
// lane l reads slot index l and cu_seqlens entries l, l + 1; a duplicate is
// a live, in-range slot that another lane also holds (every pair of lanes
// compared through lane rotations, ds_bpermute); the codes and their order
// are those of kda_validate_kernel.  Workgroup (0, 0) writes the verdict
// word.
constexpr int CHECK_IN_WAVE = 64;

// x rotated right by R + first lanes within each 16-lane row (DPP row_ror;
// a rotation by 0 is x itself), compared with s
template <int R>
__device__ __forceinline__ bool row_rotation_match(int32_t x, int32_t s)
{
    if constexpr (R == 0)
        return x == s;
    else
        return __builtin_amdgcn_mov_dpp(x, 0x120 + R, 0xF, 0xF, true) == s;
}

// any of the row rotations FIRST .. FIRST + COUNT - 1 of x matches s
template <int FIRST, int... R>
__device__ __forceinline__ bool row_rotations_match(int32_t x, int32_t s, std::integer_sequence<int, R...>)
{
    return (false | ... | row_rotation_match<FIRST + R>(x, s));
}

template <int FIRST, int COUNT>
__device__ __forceinline__ bool row_rotations_match(int32_t x, int32_t s)
{
    return row_rotations_match<FIRST>(x, s, std::make_integer_sequence<int, COUNT>{});
}

__device__ __forceinline__ int32_t wave_verdict(int32_t *verdict_word, const int32_t *slot_idx,
                                             const int32_t *cu_seqlens, int64_t num_slots, int32_t N,
                                             int64_t tokens, int64_t req, int64_t &own_slot, int64_t &bos,
                                             int64_t &eos)
{
    const int lane = threadIdx.x & 63;
    const bool mine = lane < N;
    const int at = mine ? lane : 0;   // every lane loads (the words of request 0 past N), so that the
                                      // loads issue together, without a branch between them
    const int32_t s_at = slot_idx[at];
    int32_t c0 = 0, c1 = 0;
    if (cu_seqlens) {
        c0 = cu_seqlens[at];
        c1 = cu_seqlens[at + 1];
    }
    const int32_t s = mine ? s_at : -1;
    own_slot = __builtin_amdgcn_readlane(s, (int)req);   // the workgroup's own request (req < N)
    if (cu_seqlens) {
        bos = __builtin_amdgcn_readlane(c0, (int)req);
        eos = __builtin_amdgcn_readlane(c1, (int)req);
    } else {
        bos = req * tokens;   // step calls: `tokens` is T
        eos = bos + tokens;
    }
    const bool cu_bad = cu_seqlens && mine &&
                        (c0 > c1 || (int64_t)c1 > tokens || (lane == 0 && (c0 < 0 || (int64_t)c0 > tokens)));
    const bool live = s != -1;
    const bool range_bad = live && (s < 0 || (int64_t)s >= num_slots);
    const bool checked = live && !range_bad;
    // Every pair of the first N lanes meets: lanes of one 16-lane row
    // through the row rotations of s (two lanes d apart meet at rotation d,
    // so N <= 16 needs rotations 1 .. N - 1 only), lanes of rows i and j
    // through the 16 row rotations of the copy whose rows are exchanged by
    // i ^ j (one ds_bpermute each, only for the rows that hold requests).
    // Only a live, in-range slot counts, so the -1 past N never matches.  No
    // loop: a loop keeps the compiler from sinking the kernel-argument loads
    // past it, and their wait then precedes the check (measured: about
    // 0.5 us at 32 requests).
    bool dup = false;
    if (N > 1)
        dup = row_rotations_match<1, 3>(s, s);
    if (N > 4)
        dup |= row_rotations_match<4, 4>(s, s);
    if (N > 8)
        dup |= row_rotations_match<8, 8>(s, s);
    if (N > 16)
        dup |= row_rotations_match<0, 16>(__builtin_amdgcn_ds_bpermute((lane ^ 16) << 2, s), s);
    if (N > 32) {
        dup |= row_rotations_match<0, 16>(__builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, s), s);
        dup |= row_rotations_match<0, 16>(__builtin_amdgcn_ds_bpermute((lane ^ 48) << 2, s), s);
    }
    dup &= checked;
    int32_t code = KDA_DEVICE_OK;
    if (__builtin_amdgcn_ballot_w64(cu_bad))
        code = KDA_DEVICE_ERR_CU_SEQLENS;
    if (__builtin_amdgcn_ballot_w64(dup))
        code = KDA_DEVICE_ERR_SLOT_DUP;
    if (__builtin_amdgcn_ballot_w64(range_bad))
        code = KDA_DEVICE_ERR_SLOT_RANGE;
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0)
        *verdict_word = code;
    return code;
}

// The validation verdict for a workgroup's entry check, fetched together
// with the slot index: without validation (status == nullptr) the load goes
// to the slot array's first word instead, so that no branch separates the
// two loads and one wait covers both; the value is then ignored.
__device__ __forceinline__ int32_t entry_verdict(const int32_t *status, const int32_t *slot_idx)
{
    const int32_t v = *(status ? status : slot_idx);
    return status ? v : KDA_DEVICE_OK;
}

// A workgroup's entry: the validation verdict and its request's slot index.
// VCHECK instances (validated calls of at most CHECK_IN_WAVE requests) check
// the metadata themselves, with `status` the verdict word to write, the
// launch's request count and (packed calls) token rows in preloaded
// arguments, and take the slot index and the request's token rows from the
// lanes' loads; the others read the word a kda_validate_kernel run wrote (or
// none) beside the slot, and fetch the token rows after the entry branch
// (token_rows; fetching cu_seqlens beside the slot index measured 1-3% slower
// on MI355X for the 32-column and 16-column kernels).  `tokens` is T for step
// calls (cu_seqlens == nullptr).
struct Entry {
    int32_t verdict;
    int64_t slot;
    int64_t bos, eos;   // VCHECK only
};

template <bool VCHECK>
__device__ __forceinline__ Entry entry_check(const int32_t *status, const int32_t *slot_idx,
                                             const int32_t *cu_seqlens, int64_t num_slots, int32_t requests,
                                             int64_t tokens, int64_t req)
{
    Entry e;
    if constexpr (VCHECK) {
        e.verdict = wave_verdict(const_cast<int32_t *>(status), slot_idx, cu_seqlens, num_slots, requests, tokens,
                                 req, e.slot, e.bos, e.eos);
    } else {
        e.verdict = entry_verdict(status, slot_idx);
        e.slot = slot_idx[req];
    }
    return e;
}

// The request's token rows [bos, eos): packed calls read cu_seqlens, step
// calls have T rows each.
template <bool VCHECK>
__device__ __forceinline__ void token_rows(const Entry &e, const int32_t *cu_seqlens, int64_t req, int64_t T,
                                           int64_t &bos, int64_t &eos)
{
    if constexpr (VCHECK) {
        bos = e.bos;
        eos = e.eos;
    } else if (cu_seqlens) {
        bos = cu_seqlens[req];
        eos = cu_seqlens[req + 1];
    } else {
        bos = req * T;
        eos = bos + T;
    }
}

constexpr int BODY_LOOP = 0, BODY_PEELED = 1, BODY_STAGED = 2;

// The scalars on the critical path (slot lookup -> tile address, and the
// validation verdict) come first as separate arguments: the library is built
// with kernarg preloading, so they arrive in SGPRs at wave launch and the slot
// index load issues without waiting for a kernel-argument fetch.  The rest
// travels in DecodeParams.
template <int NW, bool NORM, int BODY, bool BF16S, bool RAWG, bool VCHECK = false>
__global__ __launch_bounds__(64 * NW) void kda_decode_kernel(const int32_t *slot_idx, const int32_t *cu_seqlens,
                                                             void *state, int64_t slot_stride, int64_t num_slots,
                                                             int32_t requests, int32_t T, const int32_t *status,
                                                             DecodeParams p)
{
    static_assert(NW == 1 || NW == 2 || NW == 4, "a workgroup is 1, 2 or 4 waves");
    static_assert(!NORM || NW == 4, "the norm epilogue needs all 128 columns in one workgroup");
    constexpr int NVT = 4 / NW;   // value tiles per head

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    // grid: x = value head x value tile, y = request (no division on the way
    // to the slot index)
    const int vt = (int)(blockIdx.x % NVT);
    const int hv = (int)(blockIdx.x / NVT);
    const int64_t req = blockIdx.y;

    // slot gather: padding rows and slots outside the pool are skipped; with
    // validation, every block stops here unless the metadata check passed
    // (VCHECK packed calls carry their token rows in T)
    const Entry entry = entry_check<VCHECK>(status, slot_idx, cu_seqlens, num_slots, requests, T, req);
    const int32_t verdict = entry.verdict;
    const int64_t slot = entry.slot;
    if constexpr (BODY == BODY_LOOP)
        slot_and_token_args<RAWG>(p, slot);   // the loop body loads its first token before the tile
    if ((verdict != KDA_DEVICE_OK) | (slot < 0) | (slot >= num_slots))   // one branch: both loads first
        return;
    int64_t bos, eos;
    token_rows<VCHECK>(entry, cu_seqlens, req, T, bos, eos);
    if (eos <= bos)
        return;
    const int h = qk_head(p, hv);

    const int cg = lane & 7;              // column group: 4 columns
    const int rg = lane >> 3;             // row group: 16 key rows
    const int col = (vt * NW + wave) * 32 + cg * 4;
    const int row0 = rg * ROWS_PER_LANE;

    // The tile is streamed: read once, written once, no reuse in this call,
    // so both directions use non-temporal accesses.
    const TileIO<BF16S> tile(state, slot * slot_stride + (int64_t)hv * (KD * VD) + (int64_t)row0 * VD + col);
    f32x4 s[ROWS_PER_LANE];
    // per-token states for speculative decoding: the tile after token t
    auto keep_state = [&](int64_t t) {
        if (p.inter_state) {
            const TileIO<BF16S> it(p.inter_state, t * p.inter_stride + (int64_t)hv * (KD * VD) + (int64_t)row0 * VD + col);
#pragma unroll
            for (int i = 0; i < ROWS_PER_LANE; ++i)
                it.store(i, s[i]);
        }
    };
    TokenIn in;
    __shared__ float norm_partial[2][4];

    if constexpr (BODY == BODY_LOOP) {
        // first token's inputs, then the whole tile
        HeadGate<RAWG> hg;
        hg.load(p, hv, row0, cg);
        load_token<RAWG>(in, p, bos, h, hv, row0, col);
#pragma unroll
        for (int i = 0; i < ROWS_PER_LANE; ++i)
            s[i] = tile.load(i);
        for (int64_t t = bos; t < eos; ++t) {
            advance_token<NORM, true, RAWG>(s, in, p, hg, t, eos, h, hv, lane, wave, rg, row0, col, norm_partial);
            keep_state(t);
        }
    } else if constexpr (BODY == BODY_PEELED) {
        constexpr int FIRST_ROWS = 4;
        HeadGate<RAWG> hg;
#pragma unroll
        for (int i = 0; i < FIRST_ROWS; ++i)
            s[i] = tile.load(i);
        __builtin_amdgcn_sched_barrier(0);
        hg.load(p, hv, row0, cg);
        load_token<RAWG>(in, p, bos, h, hv, row0, col);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = FIRST_ROWS; i < ROWS_PER_LANE; ++i)
            s[i] = tile.load(i);
        // all 16 loads of the tile are in flight before any math starts
        __builtin_amdgcn_sched_barrier(0);
        advance_token<NORM, false, RAWG>(s, in, p, hg, bos, eos, h, hv, lane, wave, rg, row0, col, norm_partial);
        keep_state(bos);
        for (int64_t t = bos + 1; t < eos; ++t) {
            load_token<RAWG>(in, p, t, h, hv, row0, col);
            advance_token<NORM, false, RAWG, true>(s, in, p, hg, t, eos, h, hv, lane, wave, rg, row0, col,
                                                   norm_partial);
            keep_state(t);
        }
    } else {
        // LDS holds activated g and beta in both gate forms
        __shared__ TokenStage<NW> st;
        const HeadGate<false> no_gate;
        const int col0 = vt * NW * 32;     // first column of the workgroup's tile
        int nt = chunk_tokens(eos - bos);
        const float a_log = RAWG ? p.A_log[hv] : 0.0f;
        StagePieces<NW, RAWG> pieces;
        stage_load<NW, RAWG>(pieces, p, bos, nt, h, hv, col0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < ROWS_PER_LANE; ++i)
            s[i] = tile.load(i);
        __builtin_amdgcn_sched_barrier(0);
        const float A = RAWG ? expf(a_log) : 0.0f;
        stage_store<NW, RAWG>(st, pieces, nt, A);   // waits for the inputs only, not the tile
        if constexpr (BF16S) {
            // bf16 pool: tokens past the first chunk load their inputs directly
            // (requests that long are rare).  Without the restaging loop the
            // kernel fits in 168 VGPRs, three waves per SIMD, which the
            // half-size tiles need to keep enough bytes in flight (53.0 vs
            // 55.6 us on the packed H12 batch; the fp32 pool streams best at
            // two waves per SIMD, 69.8 vs 72.5 us the other way round).
            __syncthreads();
            for (int j = 0; j < nt; ++j) {
                read_staged(in, st.k[j], st.q[j], st.g[j], st.v[j][wave * 8 + cg], st.beta[j], rg, cg);
                advance_token<NORM, false, false>(s, in, p, no_gate, bos + j, eos, h, hv, lane, wave, rg, row0, col,
                                                  norm_partial);
                keep_state(bos + j);
            }
            if (bos + STAGE_TOKENS < eos) {
                HeadGate<RAWG> hg;
                hg.load(p, hv, row0, cg);
                for (int64_t t = bos + STAGE_TOKENS; t < eos; ++t) {
                    load_token<RAWG>(in, p, t, h, hv, row0, col);
                    advance_token<NORM, false, RAWG>(s, in, p, hg, t, eos, h, hv, lane, wave, rg, row0, col,
                                                     norm_partial);
                    keep_state(t);
                }
            }
        } else {
            for (int64_t t0 = bos; t0 < eos; t0 += STAGE_TOKENS) {
                if (t0 != bos) {
                    __syncthreads();           // every wave is done with the previous chunk
                    nt = chunk_tokens(eos - t0);
                    stage_load<NW, RAWG>(pieces, p, t0, nt, h, hv, col0);
                    stage_store<NW, RAWG>(st, pieces, nt, A);
                }
                __syncthreads();
                for (int j = 0; j < nt; ++j) {
                    read_staged(in, st.k[j], st.q[j], st.g[j], st.v[j][wave * 8 + cg], st.beta[j], rg, cg);
                    advance_token<NORM, false, false>(s, in, p, no_gate, t0 + j, eos, h, hv, lane, wave, rg, row0,
                                                      col, norm_partial);
                    keep_state(t0 + j);
                }
            }
        }
    }

    // slot scatter: the tile goes back where it came from.  The two waves of
    // a 64-column tile store together, so each 512-byte state row gets its
    // 256 bytes written at once (measured faster from 256 to 1023 tiles).
    if constexpr (NW == 2)
        __syncthreads();
#pragma unroll
    for (int i = 0; i < ROWS_PER_LANE; ++i)
        tile.store(i, s[i]);
}

// ------------------------------------------------- 16-column waves (calls with few tiles or several tokens)
//
// A second decomposition of the same arithmetic, for calls whose time goes
// into the per-token chain rather than into streaming the tile: several
// tokens per request, or few (request, value head) tiles.  A wave owns 16
// value columns x all 128 key rows; lane l holds column l % 16 of the 32 key
// rows 32 (l / 16) .. +31 (its row quarter).  The 16 lanes of a DPP row then
// share their key rows, so every per-row factor (a_i k_i, a_i q_i, a_i, k_i)
// is computed once, by the lane that owns the row pair (rows 2 (l % 16), + 1
// of the quarter), and reaches the other 15 lanes as a DPP row_newbcast
// operand of the very multiply-add that uses it: no unpacking, broadcasting
// or scaling instructions per lane and row.  Per token a lane issues 64
// fused partial-sum and 64 fused update instructions plus about 50 others
// (the 32-column layout: about 470), and twice as many waves share the work
// of a tile.  A lane's column is a 4-byte element per row, so the tile moves
// between HBM and the lanes through LDS: 16-byte accesses over full row
// pieces of the workgroup's 32 or 64 columns, then one LDS read (or write)
// per row and lane.
//
// Every result bit equals the 32-column kernel's: the lane's two 16-row
// halves are summed separately in row order and then added (the 32-column
// kernel's first reduction level), the row quarters are added by the same
// two swaps, k.q uses the same pairwise tree, and the update and readout
// are the same fused operations on the same operands.

constexpr int Q_ROWS = 32;   // key rows per lane: 128 rows over 4 row quarters

// One token's inputs as a 16-column-wave lane needs them: k, q and g of its
// row pair, v of its column, beta of the head.  With the fused gate (RAWG)
// g.x carries the row pair's raw bf16 values and beta the raw beta's bits.
struct PairIn {
    uint32_t k, q;
    float2 g;
    uint32_t v;
    float beta;
    uint32_t z;   // the norm epilogue's gate of the lane's column (NORM)
};

template <bool NORM, bool RAWG>
__device__ __forceinline__ void load_pair(PairIn &in, const DecodeParams &p, int64_t t, int h, int hv, int row0,
                                          int cp, int col)
{
    in.k = reinterpret_cast<const uint32_t *>(p.k + t * p.k_stride + h * KD + row0)[cp];
    in.q = reinterpret_cast<const uint32_t *>(p.q + t * p.q_stride + h * KD + row0)[cp];
    if constexpr (RAWG) {
        in.g.x = __uint_as_float(
            reinterpret_cast<const uint32_t *>(p.raw_gate + t * p.raw_gate_stride + (int64_t)hv * KD + row0)[cp]);
        in.beta = __uint_as_float((uint32_t)p.raw_beta[t * p.raw_beta_stride + hv]);
    } else {
        in.g = reinterpret_cast<const float2 *>(p.g + t * p.g_stride + (int64_t)hv * KD + row0)[cp];
        in.beta = p.beta[t * p.beta_stride + hv];
    }
    in.v = p.v[t * p.v_stride + (int64_t)hv * VD + col];
    if constexpr (NORM)
        in.z = p.gate[t * p.gate_stride + (int64_t)hv * VD + col];
}

// Partial sums over rows 8B .. 8B+7 of the lane's rows, whose owners are
// lanes 4B .. 4B+3 of the DPP row (lo values for even rows, hi for odd):
// u += s_i (a_i k_i), w += s_i (a_i q_i), the factor taken from its owner by
// row_newbcast.  A DPP operand must not be written by the two VALU
// instructions before it; nothing in the block writes one, and the leading
// s_nop covers whatever the compiler placed before the block.
#define Q_ROW_UW(AK, AQ, S, IMM)                                                                \
    "v_fmac_f32_dpp %0, %" AK ", %" S " row_newbcast:%c" IMM " row_mask:0xf bank_mask:0xf\n\t" \
    "v_fmac_f32_dpp %1, %" AQ ", %" S " row_newbcast:%c" IMM " row_mask:0xf bank_mask:0xf\n\t"

// The first row of a 16-row chain: the sums start from its products, in
// every lane layout (a product, not a multiply-add onto 0, so that the bits
// agree even where a product is -0).
#define Q_ROW_UW_FIRST(AK, AQ, S, IMM)                                                         \
    "v_mul_f32_dpp %0, %" AK ", %" S " row_newbcast:%c" IMM " row_mask:0xf bank_mask:0xf\n\t" \
    "v_mul_f32_dpp %1, %" AQ ", %" S " row_newbcast:%c" IMM " row_mask:0xf bank_mask:0xf\n\t"

// FIRST: rows 8B .. 8B+7 open the chain (u and w are written, not read).
template <int B, int R, bool FIRST = false>
__device__ __forceinline__ void quarter_sums8(const float (&s)[R], float ak_lo, float ak_hi, float aq_lo,
                                              float aq_hi, float &u, float &w)
{
#define Q_SUMS8_INPUTS                                                                                  \
    "v"(ak_lo), "v"(ak_hi), "v"(aq_lo), "v"(aq_hi), "v"(s[8 * B + 0]), "v"(s[8 * B + 1]),               \
        "v"(s[8 * B + 2]), "v"(s[8 * B + 3]), "v"(s[8 * B + 4]), "v"(s[8 * B + 5]), "v"(s[8 * B + 6]), \
        "v"(s[8 * B + 7]), "i"(4 * B), "i"(4 * B + 1), "i"(4 * B + 2), "i"(4 * B + 3)
    if constexpr (FIRST)
        asm volatile("s_nop 1\n\t"
                     Q_ROW_UW_FIRST("2", "4", "6", "14") Q_ROW_UW("3", "5", "7", "14")
                     Q_ROW_UW("2", "4", "8", "15") Q_ROW_UW("3", "5", "9", "15")
                     Q_ROW_UW("2", "4", "10", "16") Q_ROW_UW("3", "5", "11", "16")
                     Q_ROW_UW("2", "4", "12", "17") Q_ROW_UW("3", "5", "13", "17")
                     : "=&v"(u), "=&v"(w)
                     : Q_SUMS8_INPUTS);
    else
        asm volatile("s_nop 1\n\t"
                     Q_ROW_UW("2", "4", "6", "14") Q_ROW_UW("3", "5", "7", "14")
                     Q_ROW_UW("2", "4", "8", "15") Q_ROW_UW("3", "5", "9", "15")
                     Q_ROW_UW("2", "4", "10", "16") Q_ROW_UW("3", "5", "11", "16")
                     Q_ROW_UW("2", "4", "12", "17") Q_ROW_UW("3", "5", "13", "17")
                     : "+v"(u), "+v"(w)
                     : Q_SUMS8_INPUTS);
#undef Q_SUMS8_INPUTS
}

// The update of rows 8B .. 8B+7: s_i = k_i v' + (a_i s_i), one rounding for
// the multiply-add as in fmaf(k_i, v', a_i s_i).
#define Q_ROW_UPD(A, K, S, IMM)                                                                  \
    "v_mul_f32_dpp %" S ", %" A ", %" S " row_newbcast:%c" IMM " row_mask:0xf bank_mask:0xf\n\t" \
    "v_fmac_f32_dpp %" S ", %" K ", %12 row_newbcast:%c" IMM " row_mask:0xf bank_mask:0xf\n\t"

template <int B, int R>
__device__ __forceinline__ void quarter_update8(float (&s)[R], float a_lo, float a_hi, float k_lo, float k_hi,
                                                float vp)
{
    asm volatile("s_nop 1\n\t"
                 Q_ROW_UPD("8", "10", "0", "13") Q_ROW_UPD("9", "11", "1", "13")
                 Q_ROW_UPD("8", "10", "2", "14") Q_ROW_UPD("9", "11", "3", "14")
                 Q_ROW_UPD("8", "10", "4", "15") Q_ROW_UPD("9", "11", "5", "15")
                 Q_ROW_UPD("8", "10", "6", "16") Q_ROW_UPD("9", "11", "7", "16")
                 : "+v"(s[8 * B + 0]), "+v"(s[8 * B + 1]), "+v"(s[8 * B + 2]), "+v"(s[8 * B + 3]),
                   "+v"(s[8 * B + 4]), "+v"(s[8 * B + 5]), "+v"(s[8 * B + 6]), "+v"(s[8 * B + 7])
                 : "v"(a_lo), "v"(a_hi), "v"(k_lo), "v"(k_hi), "v"(vp),
                   "i"(4 * B), "i"(4 * B + 1), "i"(4 * B + 2), "i"(4 * B + 3));
}

// The lane's row pair of one token widened to fp32, its decay factors
// a = exp(g) and the head's beta (activated first with the fused gate).
struct PairFactors {
    float k_lo, k_hi, q_lo, q_hi, a_lo, a_hi, b;
};

template <bool RAWG>
__device__ __forceinline__ PairFactors pair_factors(const PairIn &in, const HeadGate<RAWG> &hg)
{
    PairFactors f;
    f.k_lo = bf16_lo(in.k);
    f.k_hi = bf16_hi(in.k);
    f.q_lo = bf16_lo(in.q);
    f.q_hi = bf16_hi(in.q);
    float g_lo, g_hi;
    if constexpr (RAWG) {
        const uint32_t rw = __float_as_uint(in.g.x);
        const float A = expf(hg.a_log);
        g_lo = gate_log_decay(bf16_lo(rw), hg.b.x, A);
        g_hi = gate_log_decay(bf16_hi(rw), hg.b.y, A);
        f.b = beta_from_raw(bf16_lo(__float_as_uint(in.beta)));
    } else {
        g_lo = in.g.x;
        g_hi = in.g.y;
        f.b = in.beta;
    }
    f.a_lo = __expf(g_lo);
    f.a_hi = __expf(g_hi);
    return f;
}

// The part of a token's step that does not touch the state: the factors,
// the decayed keys and queries a k and a q of the row pair, and k.q over the
// lane's ROWS key rows (the row pair, then pairs of pairs across the DPP
// row: 8 pairs for 16 rows, 16 for 32), before the sums across lanes.  A
// kernel may evaluate it for its first token while the state tile is still
// on its way.
struct PairPre {
    PairFactors f;
    float ak_lo, ak_hi, aq_lo, aq_hi;
    float kq;
};

template <int ROWS, bool RAWG>
__device__ __forceinline__ PairPre pair_pre(const PairIn &in, const HeadGate<RAWG> &hg)
{
    static_assert(ROWS == 16 || ROWS == 32, "a lane holds 16 or 32 key rows");
    PairPre r;
    r.f = pair_factors(in, hg);
    r.ak_lo = r.f.a_lo * r.f.k_lo;
    r.ak_hi = r.f.a_hi * r.f.k_hi;
    r.aq_lo = r.f.a_lo * r.f.q_lo;
    r.aq_hi = r.f.a_hi * r.f.q_hi;
    float kq = fmaf(r.f.k_hi, r.f.q_hi, r.f.k_lo * r.f.q_lo);
    kq += KDA_DPP(kq, DPP_QUAD_XOR1);
    kq += KDA_DPP(kq, DPP_QUAD_XOR2);
    kq += KDA_DPP(kq, DPP_ROW_HALF_MIRROR);
    if constexpr (ROWS == 32)
        kq += KDA_DPP(kq, DPP_ROW_MIRROR);
    r.kq = kq;
    return r;
}

// Advance the lane's column of its row quarter by one token and write its
// output (the same recurrence as advance_token).  With the norm epilogue
// (NORM, 8 waves: the workgroup holds the head's 128 columns) the sum of o^2
// is formed in the 32-column kernel's order: per group of 4 columns the
// chain fmaf(o3, o3, fmaf(o2, o2, fmaf(o1, o1, o0 o0))), which here runs
// across the group's 4 lanes by DPP row shifts; then per 32 columns the
// tree ((C0 + C7) + (C1 + C6)) + ((C2 + C5) + (C3 + C4)) over the 8 group
// sums C, and over the 4 such parts (P0 + P1) + (P2 + P3).  The group sums
// meet in LDS (norm_c, double-buffered by token parity: one barrier per
// token) and every lane evaluates the tree itself.
template <bool NORM>
__device__ __forceinline__ void advance_pair(float (&s)[Q_ROWS], const PairPre &pre, const PairIn &in,
                                             const DecodeParams &p, int64_t t, int hv, int rq, int col, int wave,
                                             int cp, float nw, float *norm_c)
{
    const float k_lo = pre.f.k_lo, k_hi = pre.f.k_hi, a_lo = pre.f.a_lo, a_hi = pre.f.a_hi, b = pre.f.b;
    const float ak_lo = pre.ak_lo, ak_hi = pre.ak_hi, aq_lo = pre.aq_lo, aq_hi = pre.aq_hi;

    // both key-axis partial sums, each 16-row half in row order
    float u_lo, w_lo, u_hi, w_hi;
    quarter_sums8<0, Q_ROWS, true>(s, ak_lo, ak_hi, aq_lo, aq_hi, u_lo, w_lo);
    quarter_sums8<2, Q_ROWS, true>(s, ak_lo, ak_hi, aq_lo, aq_hi, u_hi, w_hi);
    quarter_sums8<1>(s, ak_lo, ak_hi, aq_lo, aq_hi, u_lo, w_lo);
    quarter_sums8<3>(s, ak_lo, ak_hi, aq_lo, aq_hi, u_hi, w_hi);

    // k.q of the quarter, then the quarters
    float kq = pre.kq;
    float u = u_lo + u_hi, w = w_lo + w_hi;
    add_swaps3(kq, u, w);

    const float vp = b * (bf16_lo(in.v) - u);
    float o = p.scale * fmaf(vp, kq, w);
    quarter_update8<0>(s, a_lo, a_hi, k_lo, k_hi, vp);
    quarter_update8<1>(s, a_lo, a_hi, k_lo, k_hi, vp);
    quarter_update8<2>(s, a_lo, a_hi, k_lo, k_hi, vp);
    quarter_update8<3>(s, a_lo, a_hi, k_lo, k_hi, vp);
    if constexpr (NORM) {
        const float x1 = fmaf(o, o, KDA_DPP(o * o, DPP_ROW_SR1));
        const float x2 = fmaf(o, o, KDA_DPP(x1, DPP_ROW_SR1));
        const float x3 = fmaf(o, o, KDA_DPP(x2, DPP_ROW_SR1));   // the group sum, in lane 4m + 3
        float *part = norm_c + (t & 1) * 32;
        if (rq == 0 && (cp & 3) == 3)
            part[4 * wave + (cp >> 2)] = x3;
        __syncthreads();
        float P[4];
#pragma unroll
        for (int q32 = 0; q32 < 4; ++q32) {
            const f32x4 lo = *reinterpret_cast<const f32x4 *>(part + 8 * q32);
            const f32x4 hi = *reinterpret_cast<const f32x4 *>(part + 8 * q32 + 4);
            P[q32] = ((lo.x + hi.w) + (lo.y + hi.z)) + ((lo.z + hi.y) + (lo.w + hi.x));
        }
        const float total = (P[0] + P[1]) + (P[2] + P[3]);
        const float r = rsqrtf(fmaf(total, 1.0f / VD, p.eps));
        o = o * r * nw * silu(bf16_lo(in.z));
    }
    if (rq == 0)
        p.out[t * p.out_stride + (int64_t)hv * VD + col] = (uint16_t)pack_bf16x2(o, 0.0f);
}

// The workgroup's 128 rows x C columns of a state tile in HBM, moved with
// 16-byte non-temporal accesses over full row pieces by its THREADS lanes:
// 4 fp32 or 8 bf16 elements per lane and access, N pieces per lane.  In LDS
// the tile is fp32 either way (bf16 widened exactly on the way in, rounded
// to nearest even on the way out), row r at dword r C + 16 (r >> PAD): the
// row groups that one column read touches (32 rows apart with PAD = 5, 16
// with PAD = 4) would otherwise sit in the same banks, and the pad puts
// them 16 banks apart.
template <int C, bool BF16S, int THREADS = 4 * C, int PAD = 5>
struct SlabIO {
    static constexpr int ELEMS = BF16S ? 8 : 4;            // elements per 16-byte piece
    static constexpr int ROWS = THREADS / (C / ELEMS);     // rows per instruction
    static constexpr int N = KD / ROWS;                    // pieces per lane
    static constexpr int LDS_FLOATS = KD * C + (KD >> PAD) * 16;
    u32x4 *ptr;
    int r0, c0;

    __device__ __forceinline__ SlabIO(void *state, int64_t elem_offset, int tid)
        : r0(tid / (C / ELEMS)), c0(ELEMS * (tid % (C / ELEMS)))
    {
        ptr = reinterpret_cast<u32x4 *>(static_cast<char *>(state) +
                                        (elem_offset + (int64_t)r0 * VD + c0) * (BF16S ? 2 : 4));
    }
    static __device__ __forceinline__ int lds_at(int r, int c) { return r * C + (r >> PAD) * 16 + c; }

    __device__ __forceinline__ u32x4 load(int j) const
    {
        return __builtin_nontemporal_load(ptr + j * ROWS * VD / ELEMS);
    }
    __device__ __forceinline__ void to_lds(float *stage, int j, u32x4 w) const
    {
        float *d = stage + lds_at(j * ROWS + r0, c0);
        if constexpr (BF16S) {
            *reinterpret_cast<f32x4 *>(d) = f32x4{bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y)};
            *reinterpret_cast<f32x4 *>(d + 4) = f32x4{bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
        } else {
            *reinterpret_cast<f32x4 *>(d) = __builtin_bit_cast(f32x4, w);
        }
    }
    __device__ __forceinline__ void store_from_lds(const float *stage, int j) const
    {
        const float *d = stage + lds_at(j * ROWS + r0, c0);
        u32x4 w;
        if constexpr (BF16S) {
            const f32x4 a = *reinterpret_cast<const f32x4 *>(d), b = *reinterpret_cast<const f32x4 *>(d + 4);
            w = u32x4{pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(b.x, b.y), pack_bf16x2(b.z, b.w)};
        } else {
            w = __builtin_bit_cast(u32x4, *reinterpret_cast<const f32x4 *>(d));
        }
        __builtin_nontemporal_store(w, ptr + j * ROWS * VD / ELEMS);
    }
};

// NQ waves of 16 columns per workgroup; the norm epilogue (NORM) with 8
// waves only; fp32 or bf16 pool (BF16S); step calls (T tokens per request)
// or packed ones (cu_seqlens).  The inputs of the first PF tokens are loaded
// with the tile (later tokens, if any, load at the top of their iteration):
// after the tile's loads, or with EARLY the first token's before them (its
// kernel arguments requested with the slot index), so that its state-free
// part runs while the tile is in flight.  LDS is dynamic: the staged tile
// (C = 16 NQ columns) plus 64 floats for the norm's group sums.
template <int NQ, int PF, bool NORM, bool RAWG, bool BF16S, bool EARLY, bool VCHECK = false>
__global__ __launch_bounds__(64 * NQ) void kda_decode_q_kernel(const int32_t *slot_idx, const int32_t *cu_seqlens,
                                                               void *state, int64_t slot_stride, int64_t num_slots,
                                                               int32_t requests, int32_t T, const int32_t *status,
                                                               DecodeParams p)
{
    static_assert(NQ == 2 || NQ == 4 || NQ == 8, "a workgroup is 2, 4 or 8 waves of 16 columns");
    static_assert(!NORM || NQ == 8, "the norm epilogue needs all 128 columns in one workgroup");
    static_assert(PF >= 1 && PF <= 4, "up to 4 tokens' inputs ahead");
    static_assert(!EARLY || PF >= 2, "one-token calls load the tile first");
    constexpr int NVT = 8 / NQ;   // value tiles per head

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int vt = (int)(blockIdx.x % NVT);   // grid: x = value head x value tile, y = request
    const int hv = (int)(blockIdx.x / NVT);
    const int64_t req = blockIdx.y;

    // (VCHECK packed calls carry their token rows in T)
    const Entry entry = entry_check<VCHECK>(status, slot_idx, cu_seqlens, num_slots, requests, T, req);
    const int32_t verdict = entry.verdict;
    const int64_t slot = entry.slot;
    if constexpr (EARLY)
        slot_and_token_args<RAWG>(p, slot);
    if ((verdict != KDA_DEVICE_OK) | (slot < 0) | (slot >= num_slots))   // one branch: both loads first
        return;
    int64_t bos, eos;
    token_rows<VCHECK>(entry, cu_seqlens, req, T, bos, eos);
    if (eos <= bos)
        return;
    const int64_t ntok = eos - bos;
    const int h = qk_head(p, hv);

    const int cp = lane & 15;             // column within the wave; owner of row pair cp
    const int rq = lane >> 4;             // row quarter
    const int col = (vt * NQ + wave) * 16 + cp;
    const int row0 = rq * Q_ROWS;

    float s[Q_ROWS];
    // The tile streams through LDS with 16-byte accesses over full row
    // pieces, and each lane takes its column of 32 rows from there.
    constexpr int C = 16 * NQ;
    using Slab = SlabIO<C, BF16S>;
    extern __shared__ float stage[];        // KD * C + 64 floats, then 64 for the norm
    float *norm_c = stage + KD * C + 64;
    const Slab slab(state, slot * slot_stride + (int64_t)hv * (KD * VD) + vt * C, (int)threadIdx.x);
    // the lanes' columns back into the staged tile (every wave is done with
    // its previous contents first)
    auto stage_columns = [&]() {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < Q_ROWS; ++i)
            stage[Slab::lds_at(row0 + i, 16 * wave + cp)] = s[i];
        __syncthreads();
    };
    // per-token states leave through LDS as full row pieces too
    // (p.inter_state is uniform, so every wave reaches the barriers)
    auto keep_state = [&](int64_t t) {
        if (p.inter_state) {
            stage_columns();
            const Slab it(p.inter_state, t * p.inter_stride + (int64_t)hv * (KD * VD) + vt * C, (int)threadIdx.x);
#pragma unroll
            for (int j = 0; j < Slab::N; ++j)
                it.store_from_lds(stage, j);
        }
    };
    HeadGate<RAWG> hg;
    PairIn in[PF];
    float nw = 0.0f;
    PairPre pre0;   // the first token's state-free part, evaluated ahead (EARLY only)
    {
        // EARLY: the first token's inputs go out before the tile (loads
        // complete in order), so that its state-free part runs while the
        // tile is in flight; otherwise the tile goes out first
        if constexpr (EARLY) {
            hg.load(p, hv, row0, cp);
            load_pair<NORM, RAWG>(in[0], p, bos, h, hv, row0, cp, col);
            __builtin_amdgcn_sched_barrier(0);
        }
        u32x4 piece[Slab::N];
#pragma unroll
        for (int j = 0; j < Slab::N; ++j)
            piece[j] = slab.load(j);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (!EARLY) {
            hg.load(p, hv, row0, cp);
            load_pair<NORM, RAWG>(in[0], p, bos, h, hv, row0, cp, col);
        }
        if constexpr (NORM)
            nw = bf16_lo(p.norm_weight[col]);
        // token j, or for a request shorter than PF (packed calls) its last
        // token again: a harmless repeat that keeps the loads unconditional
#pragma unroll
        for (int j = 1; j < PF; ++j)
            load_pair<NORM, RAWG>(in[j], p, j < ntok ? bos + j : eos - 1, h, hv, row0, cp, col);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (EARLY) {
            pre0 = pair_pre<Q_ROWS>(in[0], hg);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int j = 0; j < Slab::N; ++j)
            slab.to_lds(stage, j, piece[j]);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < Q_ROWS; ++i)
        s[i] = stage[Slab::lds_at(row0 + i, 16 * wave + cp)];
    // every request here has a first token (ntok >= 1); with the tile first
    // its inputs arrive after the tile, and its state-free part is evaluated
    // where it is used (measured faster than ahead of the staging)
#pragma unroll
    for (int j = 0; j < PF; ++j) {
        if (j < ntok) {
            const PairPre pre = (EARLY && j == 0) ? pre0 : pair_pre<Q_ROWS>(in[j], hg);
            advance_pair<NORM>(s, pre, in[j], p, bos + j, hv, rq, col, wave, cp, nw, norm_c);
            keep_state(bos + j);
        }
    }
    for (int64_t t = bos + PF; t < eos; ++t) {
        load_pair<NORM, RAWG>(in[0], p, t, h, hv, row0, cp, col);
        advance_pair<NORM>(s, pair_pre<Q_ROWS>(in[0], hg), in[0], p, t, hv, rq, col, wave, cp, nw, norm_c);
        keep_state(t);
    }
    if constexpr (NQ == 2 && !BF16S && !NORM) {
        // two waves serve only one-token fp32 calls of at most 64 tiles
        // (latency-bound): each lane stores its column's 32 rows itself, as
        // the split-key kernel's tile-first launches do (N8/T1 with the
        // fused gate 3.99 vs 3.81 us through LDS and direct, N4 3.52 vs 3.44)
        float *dst = static_cast<float *>(state) + slot * slot_stride + (int64_t)hv * (KD * VD) +
                     (int64_t)row0 * VD + col;
#pragma unroll
        for (int i = 0; i < Q_ROWS; ++i)
            __builtin_nontemporal_store(s[i], dst + (int64_t)i * VD);
    } else {
        // back through LDS
        stage_columns();
#pragma unroll
        for (int j = 0; j < Slab::N; ++j)
            slab.store_from_lds(stage, j);
    }
}

// ---------------------------------------------------------------------------
// Split-key 16-column waves.  A workgroup of 4 waves holds 32 columns: two
// waves per 16 columns, one for each half of the 128 key rows, so a lane
// holds one column of one 16-row group (row group rg = 4 rh + lane / 16 of
// row half rh): half the registers and half the per-token multiply-adds of
// a kda_decode_q_kernel lane, for one LDS exchange and barrier per token,
// where the two halves' partial sums meet.  The additions are those of the
// 32-row quarters: a row group's 16-row chain is the quarter's lo or hi
// chain, row groups 2m and 2m+1 add up to quarter m by the l^16 swap (lo +
// hi, the quarter's order), quarters 0 + 1 and 2 + 3 by the l^32 swap, and
// the two halves in LDS, the quarter tree's last level; k.q the same way
// from the 8 row pairs of a row group.  So the results are bitwise those of
// the other layouts.  Lanes 8 .. 15 of a DPP row hold the same row pairs
// as lanes 0 .. 7 (the row group has 8), so their k.q tree has the same
// value without a broadcast.
constexpr int S_ROWS = 16;          // key rows per lane
constexpr int S_COLS = 32;          // columns per workgroup
constexpr int S_XCH = 3 * S_COLS;   // one row half's u, w and k.q per column

// The exchange slots of a lane (xw: the one it writes, rows 0 .. 2 only;
// xm, xo: its column's three sums of its own and of the other row half),
// in the buffer of parity 0; `buf` picks the buffer.
struct SplitXch {
    float *xw;
    const float *xm, *xo;
};

__device__ __forceinline__ void advance_split(float (&s)[S_ROWS], const PairPre &pre, const PairIn &in,
                                              const DecodeParams &p, int64_t t, int hv, int rh, int rgl, int col,
                                              const SplitXch &xs, int buf)
{
    const PairFactors &f = pre.f;
    float uh, wh;
    quarter_sums8<0, S_ROWS, true>(s, pre.ak_lo, pre.ak_hi, pre.aq_lo, pre.aq_hi, uh, wh);
    quarter_sums8<1>(s, pre.ak_lo, pre.ak_hi, pre.aq_lo, pre.aq_hi, uh, wh);
    const float sum = spread_swaps3(uh, wh, pre.kq);   // u, w, k.q of the row half in rows 0, 1, 2
    // the halves meet in LDS, double-buffered by the token's parity within
    // the request (a compile-time offset where the tokens are unrolled): a
    // buffer is written again two tokens later, after every wave has passed
    // the barrier of the token between, so after its reads of this one
    const int off = buf * (2 * S_XCH);
    if (rgl < 3)
        xs.xw[off] = sum;
    __syncthreads();
    const float u = xs.xm[off] + xs.xo[off];
    const float w = xs.xm[off + 1] + xs.xo[off + 1];
    const float kq = xs.xm[off + 2] + xs.xo[off + 2];
    const float vp = f.b * (bf16_lo(in.v) - u);
    const float o = p.scale * fmaf(vp, kq, w);
    quarter_update8<0>(s, f.a_lo, f.a_hi, f.k_lo, f.k_hi, vp);
    quarter_update8<1>(s, f.a_lo, f.a_hi, f.k_lo, f.k_hi, vp);
    if (rh == 0 && rgl == 0)
        p.out[t * p.out_stride + (int64_t)hv * VD + col] = (uint16_t)pack_bf16x2(o, 0.0f);
}

// Step calls (T tokens per request) without the norm epilogue, fp32 or bf16
// pool.  Waves 0, 1 hold row half 0 of columns 0 .. 15 and 16 .. 31 of the
// workgroup's 32, waves 2, 3 row half 1.  The tile streams in through LDS
// as in kda_decode_q_kernel (here with rows 16 apart padded to other
// banks), followed there by the exchange buffers; it goes back the same
// way, or with an fp32 pool and the tile first straight from the lanes.
//
// Workgroup placement.  The hardware hands workgroups to the 8 XCDs in turn
// (x fastest), so by default (x = value head * 4 + value tile) a head's 4
// value tiles run on 4 XCDs, each of which fetches the head's token inputs
// into its own L2.
// With HEAD_XCD the blocks of each group of 32 map to 8 heads x 4 tiles so
// that blocks b, b + 8, b + 16, b + 24 (one XCD) hold one head's tiles; the
// last group holds the remaining n < 8 heads.  Same results; measured slower
// (the re-fetched input rows come from the memory-side cache, not HBM), so
// the library never picks it and KDA_FLAG_PLACEMENT forces it.
template <int PF, bool RAWG, bool BF16S, bool EARLY, bool HEAD_XCD = false, bool VCHECK = false>
__global__ __launch_bounds__(256) void kda_decode_split_kernel(const int32_t *slot_idx, void *state,
                                                               int64_t slot_stride, int64_t num_slots, int32_t HV,
                                                               int32_t T, const int32_t *status, int32_t units,
                                                               DecodeParams p)
{
    static_assert(PF >= 1 && PF <= 4, "up to 4 tokens' inputs ahead");
    static_assert(!EARLY || PF >= 2, "one-token calls load the tile first");
    constexpr int NVT = VD / S_COLS;   // value tiles per head

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    // grid: x = value head x value tile, y = request
    int vt, hv;
    int64_t req;
    if constexpr (HEAD_XCD) {
        static_assert(NVT == 4, "a group of 32 blocks is 8 heads x 4 value tiles");
        const int64_t block = (int64_t)blockIdx.y * (HV * NVT) + blockIdx.x;   // the order of hand-out
        const int64_t group = block >> 5;
        const int r = (int)(block & 31);
        const int64_t heads = (int64_t)units - group * 8;   // heads in this group: 8, or fewer in the last
        int64_t unit;
        if (heads >= 8) {
            unit = group * 8 + (r & 7);
            vt = r >> 3;
        } else {
            const int n = (int)heads;
            unit = group * 8 + r % n;
            vt = r / n;
        }
        req = unit / HV;
        hv = (int)(unit - req * HV);
    } else {
        vt = (int)(blockIdx.x % NVT);
        hv = (int)(blockIdx.x / NVT);
        req = blockIdx.y;
    }

    // (VCHECK: the launch's requests from its head count; step calls, no cu_seqlens)
    const Entry entry = entry_check<VCHECK>(status, slot_idx, nullptr, num_slots, VCHECK ? units / HV : 0, T, req);
    const int32_t verdict = entry.verdict;
    const int64_t slot = entry.slot;
    if constexpr (EARLY)
        slot_and_token_args<RAWG>(p, slot);
    if ((verdict != KDA_DEVICE_OK) | (slot < 0) | (slot >= num_slots))   // one branch: both loads first
        return;
    const int64_t bos = req * T, eos = bos + T;
    const int h = qk_head(p, hv);

    const int cp = lane & 15;           // column within the wave
    const int rgl = lane >> 4;          // row group within the row half
    const int cw = wave & 1;            // column wave
    const int rh = wave >> 1;           // row half
    const int cl = 16 * cw + cp;        // column within the workgroup
    const int col = vt * S_COLS + cl;
    const int row0 = S_ROWS * (4 * rh + rgl);
    const int pair = cp & 7;            // row pair of the lane's row group

    float s[S_ROWS];
    using Slab = SlabIO<S_COLS, BF16S, 256, 4>;
    extern __shared__ float stage[];    // the tile, then 2 x 2 exchange buffers
    float *xch = stage + Slab::LDS_FLOATS;
    const SplitXch xs{xch + rh * S_XCH + 3 * cl + rgl, xch + rh * S_XCH + 3 * cl, xch + (rh ^ 1) * S_XCH + 3 * cl};
    const Slab slab(state, slot * slot_stride + (int64_t)hv * (KD * VD) + vt * S_COLS, (int)threadIdx.x);
    auto stage_columns = [&]() {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < S_ROWS; ++i)
            stage[Slab::lds_at(row0 + i, cl)] = s[i];
        __syncthreads();
    };
    // p.inter_state is uniform, so every wave reaches the barriers
    auto keep_state = [&](int64_t t) {
        if (p.inter_state) {
            stage_columns();
            const Slab it(p.inter_state, t * p.inter_stride + (int64_t)hv * (KD * VD) + vt * S_COLS,
                          (int)threadIdx.x);
#pragma unroll
            for (int j = 0; j < Slab::N; ++j)
                it.store_from_lds(stage, j);
        }
    };
    HeadGate<RAWG> hg;
    PairIn in[PF];
    PairPre pre0;   // the first token's state-free part, evaluated ahead (EARLY only)
    {
        // the load order as in kda_decode_q_kernel
        if constexpr (EARLY) {
            hg.load(p, hv, row0, pair);
            load_pair<false, RAWG>(in[0], p, bos, h, hv, row0, pair, col);
            __builtin_amdgcn_sched_barrier(0);
        }
        u32x4 piece[Slab::N];
#pragma unroll
        for (int j = 0; j < Slab::N; ++j)
            piece[j] = slab.load(j);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (!EARLY) {
            hg.load(p, hv, row0, pair);
            load_pair<false, RAWG>(in[0], p, bos, h, hv, row0, pair, col);
        }
#pragma unroll
        for (int j = 1; j < PF; ++j)
            load_pair<false, RAWG>(in[j], p, j < T ? bos + j : eos - 1, h, hv, row0, pair, col);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (EARLY) {
            pre0 = pair_pre<S_ROWS>(in[0], hg);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int j = 0; j < Slab::N; ++j)
            slab.to_lds(stage, j, piece[j]);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < S_ROWS; ++i)
        s[i] = stage[Slab::lds_at(row0 + i, cl)];
#pragma unroll
    for (int j = 0; j < PF; ++j) {
        if (j < T) {
            const PairPre pre = (EARLY && j == 0) ? pre0 : pair_pre<S_ROWS>(in[j], hg);
            advance_split(s, pre, in[j], p, bos + j, hv, rh, rgl, col, xs, j & 1);
            keep_state(bos + j);
        }
    }
    for (int64_t t = bos + PF; t < eos; ++t) {
        load_pair<false, RAWG>(in[0], p, t, h, hv, row0, pair, col);
        advance_split(s, pair_pre<S_ROWS>(in[0], hg), in[0], p, t, hv, rh, rgl, col, xs, (int)((t - bos) & 1));
        keep_state(t);
    }
    if constexpr (!EARLY && !BF16S) {
        // Tile-first launches (at most 191 tiles: latency-bound calls) write
        // the state back straight from the lanes: each lane stores its
        // column's 16 rows, 64-byte row pieces per 16 lanes, without the LDS
        // round trip and its two barriers.  Measured on MI355X, cold caches,
        // H = 8 (us per call, through LDS vs direct): N1/T1 3.03 vs 2.92,
        // N8/T1 3.72 vs 3.56, N16/T1 4.66 vs 4.53, N8/T4 5.12 vs 4.94, N16/T2
        // 5.09 vs 4.88; the bandwidth-bound inputs-first launches keep the
        // full row pieces (N32/T2, 256 tiles: 7.0 vs 7.6).
        float *dst = static_cast<float *>(state) + slot * slot_stride + (int64_t)hv * (KD * VD) +
                     (int64_t)row0 * VD + col;
#pragma unroll
        for (int i = 0; i < S_ROWS; ++i)
            __builtin_nontemporal_store(s[i], dst + (int64_t)i * VD);
    } else {
        stage_columns();
#pragma unroll
        for (int j = 0; j < Slab::N; ++j)
            slab.store_from_lds(stage, j);
    }
}

// Metadata check for KDA_FLAG_VALIDATE: one workgroup, lowest error code
// wins.  Duplicate live slots are found exactly with an open-addressing hash
// table of slot values in LDS (linear probing, inserts by compare-and-swap):
// inserting a value that is already there is a duplicate.  The table holds
// VALIDATE_TABLE entries and takes at most half of that per pass; a call
// with more live requests makes several passes over the slot indices, each
// inserting only the slots whose hash selects that pass.
constexpr int VALIDATE_THREADS = 1024;
constexpr int VALIDATE_TABLE = 8192;                     // 32 KiB of LDS
constexpr int VALIDATE_PER_PASS = VALIDATE_TABLE / 2;
constexpr int32_t VALIDATE_EMPTY = -1;                   // never a live slot

__device__ __forceinline__ uint32_t slot_hash(int32_t s)
{
    return (uint32_t)s * 2654435761u;   // Knuth's multiplicative hash; the table uses the top bits
}

__global__ __launch_bounds__(VALIDATE_THREADS) void kda_validate_kernel(const int32_t *slot_idx,
                                                                       const int32_t *cu_seqlens, int32_t N,
                                                                       int64_t num_slots, int64_t total_tokens,
                                                                       int32_t *status)
{
    __shared__ int32_t table[VALIDATE_TABLE];
    __shared__ int32_t verdict;
    const int tid = threadIdx.x;
    if (tid == 0)
        verdict = 0x7FFFFFFF;
    int32_t found = 0x7FFFFFFF;
    // each thread's first slot index is fetched together with the cu_seqlens
    // entries (one wait for both)
    const int32_t s_first = tid < N ? slot_idx[tid] : -1;
    if (cu_seqlens) {
        for (int i = tid; i <= N; i += VALIDATE_THREADS) {
            const int32_t c = cu_seqlens[i];
            const int32_t prev = i == 0 ? 0 : cu_seqlens[i - 1];
            const bool bad = (i == 0 ? c < 0 : prev > c) || (int64_t)c > total_tokens;
            if (bad)
                found = KDA_DEVICE_ERR_CU_SEQLENS;
        }
    }
    const uint32_t passes = (uint32_t)((N + VALIDATE_PER_PASS - 1) / VALIDATE_PER_PASS);
    for (uint32_t pass = 0; pass < passes; ++pass) {
        for (int e = tid; e < VALIDATE_TABLE; e += VALIDATE_THREADS)
            table[e] = VALIDATE_EMPTY;
        __syncthreads();
        for (int i = tid; i < N; i += VALIDATE_THREADS) {
            const int32_t s = i == tid ? s_first : slot_idx[i];
            if (s == -1)
                continue;
            if (s < 0 || (int64_t)s >= num_slots) {
                if (pass == 0)
                    found = min(found, KDA_DEVICE_ERR_SLOT_RANGE);
                continue;
            }
            const uint32_t h = slot_hash(s);
            if ((h & 0xFFFFu) % passes != pass)
                continue;
            // a pass holds about N / passes <= VALIDATE_PER_PASS values; the
            // probe stops at an empty entry or at the value itself
            uint32_t e = h >> 19;                                // 13 bits: VALIDATE_TABLE entries
            bool settled = false;
            for (int probe = 0; probe < VALIDATE_TABLE && !settled; ++probe) {
                const int32_t prev = atomicCAS(&table[e], VALIDATE_EMPTY, s);
                if (prev == s)
                    found = min(found, KDA_DEVICE_ERR_SLOT_DUP);
                settled = prev == VALIDATE_EMPTY || prev == s;
                e = (e + 1) & (VALIDATE_TABLE - 1);
            }
            if (!settled) {
                // a full table (slot values whose hashes crowd one pass):
                // compare with every other slot index instead
                for (int j = 0; j < N; ++j) {
                    if (j != i && slot_idx[j] == s) {
                        found = min(found, KDA_DEVICE_ERR_SLOT_DUP);
                        break;
                    }
                }
            }
        }
        __syncthreads();
    }
    atomicMin(&verdict, found);
    __syncthreads();
    if (tid == 0)
        *status = verdict == 0x7FFFFFFF ? KDA_DEVICE_OK : verdict;
}

// Standalone gated RMSNorm: one wave per row, 4 rows per workgroup.
__global__ __launch_bounds__(256) void kda_gated_rmsnorm_kernel(const uint16_t *x, const uint16_t *z,
                                                                const uint16_t *w, uint16_t *y,
                                                                int64_t rows, int V, float eps)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows)
        return;
    const int pairs = V / 2;
    const uint32_t *xr = reinterpret_cast<const uint32_t *>(x + row * V);
    const uint32_t *zr = reinterpret_cast<const uint32_t *>(z + row * V);
    const uint32_t *wr = reinterpret_cast<const uint32_t *>(w);
    uint32_t *yr = reinterpret_cast<uint32_t *>(y + row * V);

    float ss = 0.f;
    for (int j = lane; j < pairs; j += 64) {
        const uint32_t xw = xr[j];
        const float x0 = bf16_lo(xw), x1 = bf16_hi(xw);
        ss = fmaf(x0, x0, ss);
        ss = fmaf(x1, x1, ss);
    }
    ss += __shfl_xor(ss, 1);
    ss += __shfl_xor(ss, 2);
    ss += __shfl_xor(ss, 4);
    ss += __shfl_xor(ss, 8);
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    const float r = rsqrtf(ss / (float)V + eps);
    for (int j = lane; j < pairs; j += 64) {
        const uint32_t xw = xr[j], zw = zr[j], ww = wr[j];
        const float y0 = bf16_lo(xw) * r * bf16_lo(ww) * silu(bf16_lo(zw));
        const float y1 = bf16_hi(xw) * r * bf16_hi(ww) * silu(bf16_hi(zw));
        yr[j] = pack_bf16x2(y0, y1);
    }
}

// ------------------------------------------------------------------ launches
//
// The kernel layer's side of kda_launch.h: the device check, and the
// launch of the kernel instance a call's plan names.

std::atomic<int> g_device_kind[MAX_DEVICES];   // 0 unknown, 1 gfx950, 2 other

// Dynamic LDS of a 16-column-wave kernel with NQ waves: the staged tile
// (16 NQ columns, padded) and the norm's group sums.  At eight waves it is
// above the default 64 KiB limit, which is raised once per device, before
// the first launch (so that no attribute call happens inside a caller's
// graph capture).
constexpr size_t q_lds_bytes(int nq) { return (size_t)(KD * 16 * nq + 128) * sizeof(float); }

// The split-key kernel's: the staged tile (32 columns, rows 16 apart padded)
// and the two token parities' exchange buffers of both row halves.
constexpr size_t split_lds_bytes() { return (size_t)(KD * S_COLS + (KD / 16) * 16 + 4 * S_XCH) * sizeof(float); }

template <bool NORM, bool RAWG, bool BF16S, bool VCHECK>
bool raise_q8_lds_limit_one()
{
    const void *fns[] = {reinterpret_cast<const void *>(&kda_decode_q_kernel<8, 1, NORM, RAWG, BF16S, false, VCHECK>),
                         reinterpret_cast<const void *>(&kda_decode_q_kernel<8, 2, NORM, RAWG, BF16S, false, VCHECK>),
                         reinterpret_cast<const void *>(&kda_decode_q_kernel<8, 3, NORM, RAWG, BF16S, false, VCHECK>),
                         reinterpret_cast<const void *>(&kda_decode_q_kernel<8, 4, NORM, RAWG, BF16S, false, VCHECK>)};
    for (const void *fn : fns)
        if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)q_lds_bytes(8)) != hipSuccess)
            return false;
    if constexpr (!BF16S) {   // the inputs-first order serves fp32 pools only
        const void *early[] = {
            reinterpret_cast<const void *>(&kda_decode_q_kernel<8, 2, NORM, RAWG, false, true, VCHECK>),
            reinterpret_cast<const void *>(&kda_decode_q_kernel<8, 3, NORM, RAWG, false, true, VCHECK>),
            reinterpret_cast<const void *>(&kda_decode_q_kernel<8, 4, NORM, RAWG, false, true, VCHECK>)};
        for (const void *fn : early)
            if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)q_lds_bytes(8)) != hipSuccess)
                return false;
    }
    return true;
}

template <bool NORM, bool RAWG, bool BF16S>
bool raise_q8_lds_limit()
{
    return raise_q8_lds_limit_one<NORM, RAWG, BF16S, false>() && raise_q8_lds_limit_one<NORM, RAWG, BF16S, true>();
}

DecodeParams make_params(const kda_internal::DecodeCall &c)
{
    const kda_decode_args *a = c.args;
    DecodeParams p;
    p.q = static_cast<const uint16_t *>(a->q);
    p.k = static_cast<const uint16_t *>(a->k);
    p.v = static_cast<const uint16_t *>(a->v);
    p.g = a->g;
    p.beta = a->beta;
    p.raw_gate = static_cast<const uint16_t *>(a->raw_gate);
    p.raw_beta = static_cast<const uint16_t *>(a->raw_beta);
    p.A_log = a->A_log;
    p.dt_bias = a->dt_bias;
    p.q_stride = a->q_stride;
    p.k_stride = a->k_stride;
    p.v_stride = a->v_stride;
    p.g_stride = a->g_stride;
    p.beta_stride = a->beta_stride;
    p.raw_gate_stride = a->raw_gate_stride;
    p.raw_beta_stride = a->raw_beta_stride;
    p.HV = a->HV;
    p.T = c.T;
    p.qk_magic = c.qk_magic;
    p.qk_magic_hi = c.qk_magic_hi;
    p.scale = a->scale;
    p.eps = a->norm_eps;
    p.state = a->state;
    p.slot_idx = a->slot_idx;
    p.cu_seqlens = c.cu_seqlens;
    p.out = static_cast<uint16_t *>(a->out);
    p.gate = static_cast<const uint16_t *>(a->gate);
    p.norm_weight = static_cast<const uint16_t *>(a->norm_weight);
    p.out_stride = a->out_stride;
    p.gate_stride = a->gate_stride;
    p.num_slots = a->num_slots;
    p.slot_stride = a->slot_stride;
    p.status = c.validate ? a->device_status : nullptr;
    p.inter_state = a->inter_state;
    p.inter_stride = a->inter_stride;
    p.tokens = c.tokens;
    p.check_in_kernel = 0;
    return p;
}

// The grid of a decode launch: x = value head x value tile, y = request.  A
// call with more requests than the y dimension holds is launched in ranges
// of requests, each as a call of its own.
constexpr int64_t MAX_REQUESTS_PER_LAUNCH = 65535;

// The parameter block of the requests from r0 on: the slot indices (and
// cu_seqlens, whose token offsets stay absolute) from r0, and for step calls
// every per-token tensor from token row r0 * T.  `elem` is the pool's element
// size (per-token states).
DecodeParams request_range(const DecodeParams &p, int64_t r0, int64_t elem)
{
    DecodeParams c = p;
    c.slot_idx += r0;
    if (p.cu_seqlens) {
        c.cu_seqlens += r0;
        return c;
    }
    const int64_t t0 = r0 * p.T;
    if (t0 == 0)
        return c;
    c.q += t0 * p.q_stride;
    c.k += t0 * p.k_stride;
    c.v += t0 * p.v_stride;
    if (c.g)
        c.g += t0 * p.g_stride;
    if (c.beta)
        c.beta += t0 * p.beta_stride;
    if (c.raw_gate)
        c.raw_gate += t0 * p.raw_gate_stride;
    if (c.raw_beta)
        c.raw_beta += t0 * p.raw_beta_stride;
    c.out += t0 * p.out_stride;
    if (c.gate)
        c.gate += t0 * p.gate_stride;
    if (c.inter_state)
        c.inter_state = static_cast<char *>(c.inter_state) + t0 * p.inter_stride * elem;
    return c;
}

// The launches of `kernel` (32-column or 16-column waves) over `requests`
// requests of `tiles` value tiles per head: the preloaded scalars, then the
// parameter block.
kda_status launch(const void *kernel, const DecodeParams &p, int64_t requests, int tiles, int threads, size_t lds,
                  int64_t elem, hipStream_t stream)
{
    for (int64_t r0 = 0; r0 < requests; r0 += MAX_REQUESTS_PER_LAUNCH) {
        const int64_t n = requests - r0 < MAX_REQUESTS_PER_LAUNCH ? requests - r0 : MAX_REQUESTS_PER_LAUNCH;
        DecodeParams params = r0 ? request_range(p, r0, elem) : p;
        const int32_t *slot_idx = params.slot_idx, *cu_seqlens = params.cu_seqlens;
        void *state = params.state;
        int64_t slot_stride = params.slot_stride, num_slots = params.num_slots;
        // the metadata check of VCHECK instances reads the launch's request
        // count and, for a packed call (whose kernels do not use T), its token rows
        int32_t requests = (int32_t)n;
        int32_t T = params.check_in_kernel && cu_seqlens ? (int32_t)params.tokens : params.T;
        const int32_t *status = params.status;
        void *args[] = {&slot_idx, &cu_seqlens, &state, &slot_stride, &num_slots, &requests, &T, &status, &params};
        if (hipLaunchKernel(kernel, dim3((uint32_t)(params.HV * tiles), (uint32_t)n), dim3(threads), args, lds,
                            stream) != hipSuccess)
            return KDA_ERR_LAUNCH;
    }
    return KDA_OK;
}

// ---- the 32-column kernel: the body and the width of the plan
template <int NW, bool NORM, bool BF16S, bool RAWG, bool VCHECK>
const void *launch_wide_fn(int body)
{
    // the loop body serves only fp32 pools with activated gates (the plan's
    // rule); it is not instantiated for the other forms
    if constexpr (!BF16S && !RAWG) {
        if (body == kda_internal::BODY_LOOP)
            return reinterpret_cast<const void *>(&kda_decode_kernel<NW, NORM, BODY_LOOP, BF16S, RAWG, VCHECK>);
    }
    return body == kda_internal::BODY_STAGED
               ? reinterpret_cast<const void *>(&kda_decode_kernel<NW, NORM, BODY_STAGED, BF16S, RAWG, VCHECK>)
               : reinterpret_cast<const void *>(&kda_decode_kernel<NW, NORM, BODY_PEELED, BF16S, RAWG, VCHECK>);
}

template <int NW, bool NORM, bool BF16S, bool RAWG>
kda_status launch_wide(const DecodeParams &p, int64_t units, int body, hipStream_t s)
{
    const void *fn = launch_wide_fn<NW, NORM, BF16S, RAWG, false>(body);
    if (p.check_in_kernel)
        fn = launch_wide_fn<NW, NORM, BF16S, RAWG, true>(body);
    return launch(fn, p, units / p.HV, 4 / NW, 64 * NW, 0, BF16S ? 2 : 4, s);
}

template <bool RAWG, bool BF16S>
kda_status dispatch_wide(const DecodeParams &p, int64_t units, const kda_internal::Plan &pl, bool norm,
                         hipStream_t s)
{
    if (norm)
        return pl.waves == 4 ? launch_wide<4, true, BF16S, RAWG>(p, units, pl.body, s) : KDA_ERR_UNSUPPORTED;
    switch (pl.waves) {
    case 1: return launch_wide<1, false, BF16S, RAWG>(p, units, pl.body, s);
    case 2: return launch_wide<2, false, BF16S, RAWG>(p, units, pl.body, s);
    default: return launch_wide<4, false, BF16S, RAWG>(p, units, pl.body, s);
    }
}

// ---- 16-column waves: waves per workgroup, tokens loaded ahead (PF), order
template <int NQ, int PF, bool NORM, bool RAWG, bool BF16S>
kda_status launch_quarter(const DecodeParams &p, int64_t units, bool early, hipStream_t s)
{
    const bool check = p.check_in_kernel != 0;
    const void *fn = check ? reinterpret_cast<const void *>(&kda_decode_q_kernel<NQ, PF, NORM, RAWG, BF16S, false, true>)
                           : reinterpret_cast<const void *>(&kda_decode_q_kernel<NQ, PF, NORM, RAWG, BF16S, false>);
    if constexpr (PF >= 2 && !BF16S) {
        if (early)
            fn = check ? reinterpret_cast<const void *>(&kda_decode_q_kernel<NQ, PF, NORM, RAWG, BF16S, true, true>)
                       : reinterpret_cast<const void *>(&kda_decode_q_kernel<NQ, PF, NORM, RAWG, BF16S, true>);
    }
    return launch(fn, p, units / p.HV, 8 / NQ, 64 * NQ, q_lds_bytes(NQ), BF16S ? 2 : 4, s);
}

template <int NQ, bool NORM, bool RAWG, bool BF16S>
kda_status dispatch_quarter_tokens(const DecodeParams &p, int64_t units, bool early, hipStream_t s)
{
    switch (p.cu_seqlens ? 4 : p.T) {
    case 1: return launch_quarter<NQ, 1, NORM, RAWG, BF16S>(p, units, early, s);
    case 2: return launch_quarter<NQ, 2, NORM, RAWG, BF16S>(p, units, early, s);
    case 3: return launch_quarter<NQ, 3, NORM, RAWG, BF16S>(p, units, early, s);
    default: return launch_quarter<NQ, 4, NORM, RAWG, BF16S>(p, units, early, s);
    }
}

template <bool RAWG, bool BF16S>
kda_status dispatch_quarter(const DecodeParams &p, int64_t units, const kda_internal::Plan &pl, bool norm,
                            hipStream_t s)
{
    if (norm)
        return pl.waves == 8 ? dispatch_quarter_tokens<8, true, RAWG, BF16S>(p, units, pl.early, s)
                             : KDA_ERR_UNSUPPORTED;
    if (pl.waves == 2) {
        // two waves serve only one-token fp32 calls with the fused gate
        if constexpr (RAWG && !BF16S) {
            if (p.T == 1 && !p.cu_seqlens)
                return launch_quarter<2, 1, false, true, false>(p, units, false, s);
        }
        return KDA_ERR_UNSUPPORTED;
    }
    return pl.waves == 8 ? dispatch_quarter_tokens<8, false, RAWG, BF16S>(p, units, pl.early, s)
                         : dispatch_quarter_tokens<4, false, RAWG, BF16S>(p, units, pl.early, s);
}

// ---- split-key waves (step calls only)
template <int PF, bool RAWG, bool BF16S>
kda_status launch_split(const DecodeParams &p, int64_t units, bool early, bool head_xcd, hipStream_t s)
{
    // (the head-per-XCD placement is not combined with the check in the
    // kernel: launch_decode runs kda_validate_kernel for such calls)
    const bool check = p.check_in_kernel != 0;
    const void *fn = check ? reinterpret_cast<const void *>(&kda_decode_split_kernel<PF, RAWG, BF16S, false, false, true>)
                           : reinterpret_cast<const void *>(&kda_decode_split_kernel<PF, RAWG, BF16S, false>);
    if constexpr (PF >= 2 && !BF16S) {
        if (early)
            fn = check ? reinterpret_cast<const void *>(&kda_decode_split_kernel<PF, RAWG, BF16S, true, false, true>)
                       : reinterpret_cast<const void *>(&kda_decode_split_kernel<PF, RAWG, BF16S, true>);
        if (head_xcd)
            fn = early ? reinterpret_cast<const void *>(&kda_decode_split_kernel<PF, RAWG, BF16S, true, true>)
                       : reinterpret_cast<const void *>(&kda_decode_split_kernel<PF, RAWG, BF16S, false, true>);
    }
    // the preloaded scalars (no cu_seqlens: step calls only), the launch's
    // head count, then the parameter block; requests in ranges as in launch()
    const int64_t requests = units / p.HV;
    for (int64_t r0 = 0; r0 < requests; r0 += MAX_REQUESTS_PER_LAUNCH) {
        const int64_t n = requests - r0 < MAX_REQUESTS_PER_LAUNCH ? requests - r0 : MAX_REQUESTS_PER_LAUNCH;
        DecodeParams params = r0 ? request_range(p, r0, BF16S ? 2 : 4) : p;
        const int32_t *slot_idx = params.slot_idx;
        void *state = params.state;
        int64_t slot_stride = params.slot_stride, num_slots = params.num_slots;
        int32_t HV = params.HV, T = params.T, heads = (int32_t)(n * HV);
        const int32_t *status = params.status;
        void *args[] = {&slot_idx, &state, &slot_stride, &num_slots, &HV, &T, &status, &heads, &params};
        if (hipLaunchKernel(fn, dim3((uint32_t)(HV * (VD / S_COLS)), (uint32_t)n), dim3(256), args,
                            split_lds_bytes(), s) != hipSuccess)
            return KDA_ERR_LAUNCH;
    }
    return KDA_OK;
}

template <bool RAWG, bool BF16S>
kda_status dispatch_split(const DecodeParams &p, int64_t units, bool early, bool head_xcd, hipStream_t s)
{
    if (p.cu_seqlens || (head_xcd && (p.T < 2 || BF16S)))
        return KDA_ERR_UNSUPPORTED;
    switch (p.T) {
    case 1: return launch_split<1, RAWG, BF16S>(p, units, false, false, s);
    case 2: return launch_split<2, RAWG, BF16S>(p, units, early, head_xcd, s);
    case 3: return launch_split<3, RAWG, BF16S>(p, units, early, head_xcd, s);
    default: return launch_split<4, RAWG, BF16S>(p, units, early, head_xcd, s);
    }
}

template <bool RAWG, bool BF16S>
kda_status dispatch(const DecodeParams &p, int64_t units, const kda_internal::Plan &pl, bool norm, hipStream_t s)
{
    switch (pl.kernel) {
    case kda_internal::KERNEL_WIDE: return dispatch_wide<RAWG, BF16S>(p, units, pl, norm, s);
    case kda_internal::KERNEL_QUARTER: return dispatch_quarter<RAWG, BF16S>(p, units, pl, norm, s);
    case kda_internal::KERNEL_SPLIT: return norm ? KDA_ERR_UNSUPPORTED : dispatch_split<RAWG, BF16S>(p, units, pl.early, pl.head_xcd, s);
    }
    return KDA_ERR_UNSUPPORTED;
}

}  // namespace

namespace kda_internal {

kda_status device_ready()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES)
        return KDA_ERR_DEVICE;
    int kind = g_device_kind[dev].load(std::memory_order_relaxed);
    if (kind == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return KDA_ERR_DEVICE;
        kind = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        if (kind == 1) {
            const bool raised = raise_q8_lds_limit<false, false, false>() && raise_q8_lds_limit<false, false, true>() &&
                                raise_q8_lds_limit<false, true, false>() && raise_q8_lds_limit<false, true, true>() &&
                                raise_q8_lds_limit<true, false, false>() && raise_q8_lds_limit<true, false, true>() &&
                                raise_q8_lds_limit<true, true, false>() && raise_q8_lds_limit<true, true, true>();
            if (!raised)
                return KDA_ERR_DEVICE;
        }
        g_device_kind[dev].store(kind, std::memory_order_relaxed);
    }
    return kind == 1 ? KDA_OK : KDA_ERR_DEVICE;
}

kda_status launch_decode(const DecodeCall &c)
{
    DecodeParams p = make_params(c);
    const kda_decode_args *a = c.args;
    hipStream_t s = static_cast<hipStream_t>(c.stream);
    if (c.validate && a->N <= CHECK_IN_WAVE && !c.plan.head_xcd && c.tokens <= 0x7FFFFFFF) {
        // the waves of the decode check the metadata themselves (the VCHECK
        // instances, `status` the word they write): no second launch
        p.check_in_kernel = 1;
    } else if (c.validate) {
        const int32_t *slots = a->slot_idx;
        const int32_t *cu = c.cu_seqlens;
        int32_t n = a->N;
        int64_t num_slots = a->num_slots, tokens = c.tokens;
        int32_t *status = a->device_status;
        void *vargs[] = {&slots, &cu, &n, &num_slots, &tokens, &status};
        if (hipLaunchKernel(reinterpret_cast<const void *>(&kda_validate_kernel), dim3(1), dim3(VALIDATE_THREADS),
                            vargs, 0, s) != hipSuccess)
            return KDA_ERR_LAUNCH;
    }
    const int64_t units = (int64_t)a->N * a->HV;
    const bool norm = a->gate != nullptr;
    const bool raw = a->raw_gate != nullptr;
    if (c.bf16_state)
        return raw ? dispatch<true, true>(p, units, c.plan, norm, s) : dispatch<false, true>(p, units, c.plan, norm, s);
    return raw ? dispatch<true, false>(p, units, c.plan, norm, s) : dispatch<false, false>(p, units, c.plan, norm, s);
}

kda_status launch_gated_rmsnorm(const void *x, const void *gate, const void *weight, void *y, int64_t rows,
                                int32_t V, float eps, void *stream)
{
    const int64_t blocks = (rows + 3) / 4;
    const uint16_t *xp = static_cast<const uint16_t *>(x);
    const uint16_t *zp = static_cast<const uint16_t *>(gate);
    const uint16_t *wp = static_cast<const uint16_t *>(weight);
    uint16_t *yp = static_cast<uint16_t *>(y);
    int Vi = V;
    void *args[] = {&xp, &zp, &wp, &yp, &rows, &Vi, &eps};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&kda_gated_rmsnorm_kernel),
                                         dim3((uint32_t)blocks), dim3(256), args, 0, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

}  // namespace kda_internal
