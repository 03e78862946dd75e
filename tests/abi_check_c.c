/* C side of tests/abi_check.cpp: a C caller may pass any int where the status enum is
 * expected (in C an enum is an integer type), which C++ cannot express without undefined
 * behaviour. */
#include "w4a16.h"

const char* abi_check_status_string_of_int(int v) { return w4a16_status_string(v); }
