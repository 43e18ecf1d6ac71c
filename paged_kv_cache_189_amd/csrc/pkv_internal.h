// Internal declarations shared by the C ABI and the block manager of libpkv.
// Not part of the public interface.  No HIP dependency.
#pragma once

#include <string>

#include "../../include/pkv.h"

// Records `msg` as the calling thread's last error and returns `s`.
pkv_status pkv_fail(pkv_status s, const std::string& msg);
