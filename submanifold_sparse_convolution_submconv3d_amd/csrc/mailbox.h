// Device side of the status mailbox (struct Mailbox, common.h): a kernel that ends a
// call posts the call's status to pinned host memory, which the host polls.
#pragma once

#include "common.h"

namespace sc {

// The status into the host's pinned mailbox, `seq` last (one thread): a system-scope
// release first, so the host sees the status only after every write before it.
__device__ __forceinline__ void mailbox_post(Mailbox *mb, uint32_t seq, uint32_t flags, unsigned long long taps,
                                             unsigned long long count)
{
    mb->flags = flags;
    mb->taps = taps;
    mb->count = count;
    __threadfence_system();
    __hip_atomic_store(&mb->seq, seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
}

}  // namespace sc
