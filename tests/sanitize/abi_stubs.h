// abi_stubs.h -- what the stand-in launchers of abi_stubs.cpp record.
#pragma once

#include "fa_internal.h"

namespace stub {
struct Record {
    const char *kernel = nullptr;
    int calls = 0;
    int scratch_lookups = 0;
    fa::FwdArgs fwd{};
    fa::DecodeArgs dec{};
    fa::BwdArgs bwd{};
};
extern Record last;
}  // namespace stub
