// Internal declarations of the host-CPU decode attention (attn_host.cpp):
// plain C++, no HIP, so the HIP translation units and the host-only one can
// both include it.  Not part of the C ABI (see include/fg.h for that).
#pragma once

#include <cstddef>
#include <cstdint>
#include <functional>

#include "../../include/fg.h"

namespace fg {

int set_error(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
int check_dims(const fg_dims* d);

// A fixed set of worker threads that run one parallel loop at a time; the
// calling thread works too.  run() returns when every item is done.
class HostPool {
   public:
    // n: threads in all, the caller included (<= 0: the hardware's count)
    explicit HostPool(int n);
    ~HostPool();
    HostPool(const HostPool&) = delete;
    HostPool& operator=(const HostPool&) = delete;
    int threads() const { return nthreads_; }
    // f(begin, end) over [0, items) in chunks, on every thread; returns when
    // all are done.  Threads that could not be started are simply missing.
    void run(int64_t items, const std::function<void(int64_t, int64_t)>& f);

   private:
    struct State;
    State* s_;
    int nthreads_;
};

// Attention of sequences seq0 .. seq0 + nseq - 1 of an fp16 or 4-bit host
// cache at position pos (rows < pos from the cache, the current token from
// its fresh k, v), out fp16 [nseq, h1]; qkv: fp16 rows of ld elements, q at
// column 0, k at h1, v at 2 h1.  append: also store k, v at row pos (4-bit:
// quantized as the device codec does).  Arguments are checked by the caller.
// Returns FG_OK, or FG_ERR_CAPACITY (error text set) when a thread's score
// buffer could not be allocated; that thread's items are then not computed.
int host_attn_decode(const uint16_t* qkv, int64_t ld, const fg_kv* kv, int32_t seq0, int32_t nseq,
                         const fg_dims* d, int32_t pos, bool append, uint16_t* out, HostPool& pool);

// Argument checks of the host attention entry points (also used by the layer
// path): dims, pointers, either cache format, sequences, pos and ld.
int check_host_attn(const void* qkv, int64_t ld, const fg_kv* kv, int32_t seq0, int32_t nseq,
                    const fg_dims* d, int32_t pos, const void* out);

}  // namespace fg
