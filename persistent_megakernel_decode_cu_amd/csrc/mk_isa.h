// mk_isa.h - instruction encoding, event table and on-chip layout shared by
// the host scheduler (mk_sched.cpp) and the resident interpreter
// (mk_kernels.hip).
//
// "Inference MegaKernel" (shaojiemike.top), section "hand-written whole-model
// MegaKernel / principle, schedule and dataflow": each compute unit owns a
// queue of fixed-width int32 instructions ([S, Q, 32] in its object table);
// an instruction names its op body, the counters it waits on and the
// counters it bumps when done. Here a wait or a bump names an *event*; the
// event table maps it to one counter and the count it must reach per step.
#pragma once
#include <stdint.h>

namespace mk {

// op bodies: the page's RMS_NORM is fused into every consumer of a norm
// (QKV, UPGATE, LMHEAD recompute it from the residual stream), RoPE and the
// K/V append live in ATTN, and the O projection with its residual is its own
// body (the page's op list has no O opcode; "residual" is in its op chain).
enum Op : int32_t {
    OP_END = 0,
    OP_QKV = 1,     // rows [r0,r1) of Wqkv . rmsnorm(x)               -> qkv
    OP_ATTN = 2,    // request b, kv head g, K/V chunk c of nch        -> partials, merged by the last chunk
    OP_OPROJ = 3,   // rows [r0,r1) of Wo . o, plus residual            -> x
    OP_UPGATE = 4,  // rows [r0,r1) of Wgate, Wup . rmsnorm(x), SiLU    -> act
    OP_DOWN = 5,    // rows [r0,r1) of Wdown . act, plus residual       -> x
    OP_LMHEAD = 6,  // rows [r0,r1) of E . rmsnorm_final(x), argmax     -> logits, partial argmax
    OP_COUNT = 7
};

// instruction words
enum : int {
    W_OP = 0,
    W_LAYER = 1,
    W_R0 = 2,
    W_R1 = 3,
    W_B = 4,
    W_G = 5,
    W_C = 6,
    W_NCH = 7,
    W_FLAGS = 8,
    W_NWAIT = 9,
    W_WAIT = 10,   // MAX_WAIT event ids
    W_NPUB = 18,
    W_PUB = 19,    // MAX_PUB event ids
    W_MERGE = 23,  // event whose counter elects the last finisher (-1: none)
    W_SLOT = 24,   // this instruction's slot among the merge's partials
    W_NSLOT = 25,  // slots of the merge
    W_SEQ = 26,    // position in the global topological order
    INSTR_WORDS = 32,
    MAX_WAIT = 8,
    MAX_PUB = 4
};

enum : int32_t {
    F_X_FROM_INPUT = 1,  // layer 0: residual stream comes from the embedding row / hidden_in
    F_WRITE_HIDDEN = 2,  // last layer's DOWN: also write hidden_out
    F_STEP_FINAL = 4     // the merge finisher of this instruction ends the step
};

// event table: EV_WORDS int32 per event
enum : int { EV_CTR = 0, EV_NEED = 1, EV_KIND = 2, EV_WORDS = 16 };
enum : int32_t { EVK_WAIT = 0, EVK_MERGE = 1 };
// counters are spaced one 128-byte line apart
constexpr int CTR_STRIDE = 32;

constexpr int GRANULE = 1024;       // bytes moved by one wave-wide 16-byte-per-lane DMA
constexpr int WAVE = 64;
constexpr int N_COMPUTE_WAVES = 8;
constexpr int N_WAVES = N_COMPUTE_WAVES + 2;   // + loader + poller
constexpr int BLOCK_THREADS = N_WAVES * WAVE;
constexpr int LDS_LIMIT = 160 * 1024;          // gfx950 LDS per workgroup
constexpr int MISC_BYTES = 4096;
constexpr int ATTN_PART = 64 + 2;              // o[d], m, l of one head
constexpr int MAX_B = 8;
constexpr int MAX_G = 8;

// device error word: code << 28 | cu << 16 | pc
enum : int32_t { ERR_TIMEOUT = 1, ERR_OPCODE = 2, ERR_RANGE = 3, ERR_NAN = 4 };

}  // namespace mk
