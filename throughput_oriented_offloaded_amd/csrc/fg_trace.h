// Internal tracing hooks (see trace.hip).  A TraceScope placed around a kernel
// launch records one event before and one after it on the same stream when
// tracing is enabled; otherwise it does nothing.  A second kind (kind2 >= 0)
// credits the same bracket to that kind too (a decoder projection beside the
// GEMM kind), so no bracket is ever nested inside another and timed with it.
#pragma once

#include "fg_internal.h"

namespace fg {

enum TraceKind {
    TK_QUANT = 0, TK_DEQUANT, TK_GEMM_Q4, TK_GEMM_F16, TK_SPLITK_REDUCE, TK_ATTN_DECODE_Q4,
    TK_ATTN_DECODE_F16, TK_KV_STORE, TK_ATTN_PREFILL, TK_LAYERNORM, TK_EMBED, TK_ARGMAX,
    TK_REDUCE_LN, TK_ATTN_TOPK_Q4, TK_ATTN_TOPK_F16, TK_KV_H2D, TK_KV_D2H, TK_W_H2D,
    TK_PROJ_QKV, TK_PROJ_OUT, TK_PROJ_FC1, TK_PROJ_FC2, TK_COUNT
};

bool trace_on();

// Marks a TraceScope whose launch records the two events itself: the kernel is
// launched with hipExtLaunchKernelGGL and the events that trace_take_ext hands
// out, so they hold the kernel's own start and end, and no event packet sits
// between it and its neighbours (an event pair recorded around a launch drains
// the queue before and after it: about 5 us of idle time per pair).  A scope
// in this mode whose events no launch takes is dropped.
struct ExtLaunch {};
constexpr ExtLaunch kExtLaunch{};

class TraceScope {
  public:
    TraceScope(int kind, hipStream_t st, double flops, double bytes, int kind2 = -1);
    TraceScope(ExtLaunch, int kind, hipStream_t st, double flops, double bytes, int kind2 = -1);
    ~TraceScope();
    TraceScope(const TraceScope&) = delete;
    TraceScope& operator=(const TraceScope&) = delete;

  private:
    hipStream_t st_ = nullptr;
    long idx_ = -1;
    bool ext_ = false;
};

// The events of this thread's innermost pending launch-recorded scope (and
// that scope is then no longer pending); null events when there is none, in
// which case hipExtLaunchKernelGGL launches without timing.
void trace_take_ext(hipEvent_t* start, hipEvent_t* stop);

}  // namespace fg
